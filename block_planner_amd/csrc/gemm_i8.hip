// gemm_i8.hip -- the linear on the int8 matrix cores, for weight tiles whose
// blocks are all INT8 (prefill): y[m, n] = sum over K-blocks kb of
// s[n, kb] * (sum_i q[n, 64kb+i] * x_hat[m, 64kb+i]) with exact int32 block
// sums (HyperTensor 1.0.1 page, intro: the fused kernels run the plan's
// mixed precisions; "Key Features": HyperLinear).
//
// The page fixes no integer encoding of the activations.  x is encoded per
// token (row) m as two int8 planes with a power-of-two scale:
//   amax = max_k |x[m, k]| = f * 2^E, f in [0.5, 1);
//   v = round_half_even(x * 2^(14-E)),  |v| <= 2^14 (exact for bfloat16 x);
//   hi = floor((v + 128) / 256) in [-64, 64],  lo = v - 256 * hi;
//   x_hat = v * 2^(E-14), within 2^-14 * amax of x.
// A row holding Inf or NaN gets a NaN scale (its outputs in these tiles are
// NaN); an all-zero row has scale 1 and zero planes.  Per K-block the two
// planes give exact int32 sums Ch, Cl (v_mfma_i32_16x16x64_i8, one 64-deep
// block per instruction), combined exactly as 256 * Ch + Cl, converted to
// fp32 and added to the accumulator times the block's weight scale; the row's
// scale 2^(E-14) multiplies the finished sum (exact).
//
// Work split: a 256-column weight tile (16 row tiles of 16) over one K-split
// qualifies when all of its blocks are INT8; the bfloat16 MFMA kernel of the
// same call skips exactly those columns, so each output is written once.  In
// a qualifying tile the INT8 blocks of one K-step are 16 consecutive blocks
// per row tile (packed in (kb, row) order), i.e. one contiguous 1 KiB operand
// per 16 columns.
//
// Kernels:
//   xq_kernel       one workgroup per row of x: the row maximum, then the
//                   planes, written in MFMA operand order ([16-row group][kb]
//                   [plane][lane][16 bytes], lane = row + 16 * (entry / 16));
//   gemm_i8_kernel  a workgroup owns a 128 x 256 tile of y over one K-split;
//                   its eight wavefronts copy the next steps' operands
//                   straight from memory into LDS (global_load_lds, four
//                   stages) and each runs the MFMAs of a 64 x 64 sub-tile.
//                   The wide tile matters: per K-step it copies 33 KiB for
//                   4.2 MFLOP, where a 256 x 64 tile copies 37 KiB for 2.1.
#include "int8_tile.h"
#include "linear_host.h"

namespace ht {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kI8Threads = 512;            // 8 wavefronts
constexpr int64_t kI8ChunkRows = 8192;          // rows of x per launch (bounds the planes' workspace)

// s_waitcnt immediate: wait until at most n vector-memory operations of this
// wavefront are outstanding (no wait on the other counters).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

struct XqArgs {
    const uint16_t *x;
    int64_t ldx;
    uint32_t M, KB;
    uint8_t *q;         // planes [G][KB][2][64][16]
    float *rs;          // row scales [G * 16]
};

// One workgroup per row m of x: the row's maximum |x| (and whether it holds
// an Inf or NaN), then its entries as the two planes.  Rows past M in the
// last 16-row group are left unwritten: they only feed outputs that are not
// stored.  Consecutive workgroup indices go to different XCDs in turn, so the
// index is permuted (when the grid is a multiple of 8) such that each XCD
// writes whole 16-row groups: the rows of a group share cache lines.
__global__ __launch_bounds__(256) void xq_kernel(XqArgs a) {
    __shared__ float smax[4];
    __shared__ uint32_t sbad[4];
    uint32_t m = blockIdx.x;
    if ((gridDim.x & 7u) == 0) m = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const uint32_t t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const uint32_t K = a.KB * 64u;
    const uint16_t *row = a.x + int64_t(m) * a.ldx;
    float amax = 0.0f;
    uint32_t bad = 0;
    for (uint32_t p = t; p < K / 8u; p += 256u) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + 8u * p);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float f0 = fabsf(__uint_as_float(u[i] << 16));
            const float f1 = fabsf(__uint_as_float(u[i] & 0xFFFF0000u));
            bad |= !(f0 <= 3.4028235e38f) || !(f1 <= 3.4028235e38f);   // Inf or NaN
            amax = fmaxf(amax, fmaxf(f0, f1));
        }
    }
    amax = fmaxf(amax, dpp_f32<kDppXor1>(amax));
    amax = fmaxf(amax, dpp_f32<kDppXor2>(amax));
    amax = fmaxf(amax, dpp_f32<kDppHalfMirror>(amax));
    amax = fmaxf(amax, dpp_f32<kDppMirror>(amax));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    bad = __any(bad != 0u) ? 1u : 0u;
    if (lane == 0) {
        smax[wv] = amax;
        sbad[wv] = bad;
    }
    __syncthreads();
    amax = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
    bad = sbad[0] | sbad[1] | sbad[2] | sbad[3];
    int E = 0;
    if (amax > 0.0f) (void)frexpf(amax, &E);
    const int sh = amax > 0.0f ? 14 - E : 0;
    if (t == 0) a.rs[m] = bad ? __builtin_nanf("") : amax > 0.0f ? ldexpf(1.0f, E - 14) : 1.0f;
    // planes: piece p = entries [16p, +16) -> K-block p / 4, lane r + 16 (p % 4)
    const uint32_t g = m >> 4, r = m & 15;
    for (uint32_t p = t; p < K / 16u; p += 256u) {
        const uint32_t kb = p >> 2, qq = p & 3u;
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
        if (!bad) {
            v0 = *reinterpret_cast<const uint4 *>(row + 16u * p);
            v1 = *reinterpret_cast<const uint4 *>(row + 16u * p + 8u);
        }
        const uint32_t u[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        uint32_t hw[4] = {0, 0, 0, 0}, lw[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t bits = (i & 1) ? (u[i >> 1] & 0xFFFF0000u) : (u[i >> 1] << 16);
            const int32_t iv = int32_t(rintf(ldexpf(__uint_as_float(bits), sh)));
            const int32_t h = (iv + 128) >> 8;   // arithmetic shift: floor
            const int32_t lo = iv - h * 256;
            hw[i >> 2] |= (uint32_t(h) & 0xFFu) << (8 * (i & 3));
            lw[i >> 2] |= (uint32_t(lo) & 0xFFu) << (8 * (i & 3));
        }
        uint8_t *dst = a.q + ((uint64_t(g) * a.KB + kb) * 2u) * 1024u + 16u * (r + 16u * qq);
        *reinterpret_cast<uint4 *>(dst) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4 *>(dst + 1024) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
}

// W8A8 encoding of x (HT_PATH_W8A8): per token m and 64-wide K-block kb, one
// int8 code per entry and one power-of-two scale:
//   amax = max over the block of |x| = f * 2^E, f in [0.5, 1);
//   q = clamp(round_half_even(x * 2^(7-E)), -127, 127);
//   scale 2^(E-7) (1 for an all-zero block, NaN for a block holding an Inf
//   or NaN, whose codes are 0).
// One workgroup per row of x; wavefront v encodes K-blocks v, v + 4, ...,
// lane l entry l.  Codes go to the same operand order as the two-plane
// encoding ([16-row group][kb][lane = row + 16 * (entry / 16)][16 bytes]),
// one plane; the scales to [kb][16 * groups] (contiguous per K-block, as
// the matrix-core kernel copies them).
struct Xq8Args {
    const uint16_t *x;
    int64_t ldx;
    uint32_t M, KB, Mp;   // Mp = 16 * groups
    uint8_t *q;           // codes [G][KB][64][16]
    float *sx;            // block scales [KB][Mp]
};

__global__ __launch_bounds__(256) void xq8_kernel(Xq8Args a) {
    uint32_t m = blockIdx.x;
    if ((gridDim.x & 7u) == 0) m = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const uint32_t t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const uint16_t *row = a.x + int64_t(m) * a.ldx;
    const uint32_t g = m >> 4, r = m & 15;
    for (uint32_t kb = wv; kb < a.KB; kb += 4u) {
        const float f = __uint_as_float(uint32_t(row[64u * kb + lane]) << 16);
        const float af = fabsf(f);
        const bool bad = !(af <= 3.4028235e38f);   // Inf or NaN
        float amax = bad ? 0.0f : af;
        amax = fmaxf(amax, dpp_f32<kDppXor1>(amax));
        amax = fmaxf(amax, dpp_f32<kDppXor2>(amax));
        amax = fmaxf(amax, dpp_f32<kDppHalfMirror>(amax));
        amax = fmaxf(amax, dpp_f32<kDppMirror>(amax));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const bool anybad = __any(bad);
        int E = 0;
        if (amax > 0.0f) (void)frexpf(amax, &E);
        const int sh = amax > 0.0f ? 7 - E : 0;
        float v = anybad ? 0.0f : rintf(ldexpf(f, sh));
        v = fminf(127.0f, fmaxf(-127.0f, v));
        const uint32_t code = uint32_t(int32_t(v)) & 0xFFu;
        const uint32_t word = code | (uint32_t(__shfl_down(int(code), 1)) << 8) |
                              (uint32_t(__shfl_down(int(code), 2)) << 16) | (uint32_t(__shfl_down(int(code), 3)) << 24);
        if ((lane & 3u) == 0u) {
            uint8_t *dst = a.q + (uint64_t(g) * a.KB + kb) * 1024u + 16u * (r + 16u * (lane >> 4)) + 4u * ((lane & 15u) >> 2);
            *reinterpret_cast<uint32_t *>(dst) = word;
        }
        if (lane == 0)
            a.sx[uint64_t(kb) * a.Mp + m] = anybad ? __builtin_nanf("") : amax > 0.0f ? ldexpf(1.0f, E - 7) : 1.0f;
    }
}

struct I8Args {
    LayerDev w;
    const uint8_t *q;         // x planes
    const float *rs;          // x row scales (two-plane encoding), or
    const float *sx;          // x block scales [KB][Mp] (W8A8 encoding)
    uint32_t Mp;
    float *y;                 // fp32 output, or
    uint16_t *ybf;            // bfloat16 output (round to nearest even), or
    float *partial;           // per-split partial sums [S][M][N] (no activation)
    int64_t ldy;
    uint32_t M, G;            // rows of x, 16-row groups of the planes
    uint32_t KBs;             // K-blocks per split
    uint32_t MT, NT;          // row tiles of x (128 rows), weight tiles (256 rows)
    int act;
};

// 16-byte (resp. 4-byte) copy per lane from global memory straight into LDS
// at dst + 16 * lane (resp. 4 * lane).  Issued as inline assembly so that the
// compiler adds no waits for them; the kernel waits with vm_wait.
__device__ __forceinline__ void lds_copy16(const void *src, const void *dst) {
    const uint32_t d = uint32_t(uintptr_t((__attribute__((address_space(3))) const uint8_t *)(dst)));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(d) : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const void *src, const void *dst) {
    const uint32_t d = uint32_t(uintptr_t((__attribute__((address_space(3))) const uint8_t *)(dst)));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(src), "s"(d) : "memory", "m0");
}

// Workgroup (mt, it, split) owns rows [128*mt, +128) of x and weight rows
// [256*it, +256) over K-blocks [KBs*split, +KBs) (consecutive workgroup
// indices go to different XCDs in turn, so the index is permuted such that
// each XCD gets a contiguous run of tiles, mostly one row tile of x, which its
// L2 then serves to all of them); it returns at once unless that weight tile
// is all INT8 over the split.  Wavefront w owns rows [64 (w / 4), +64) and
// columns [64 (w % 4), +64) of the tile: 4 x 4 output tiles of 16 x 16.
//
// LDS stage (one K-step): the x planes of the 128 rows (8 groups x 2 planes x
// 1 KiB, operand order), the weight codes (16 x 1 KiB, operand order: lane l
// -> weight row l % 16 of the row tile, entries [16 (l / 16), +16)) and the
// 256 column scales.  Wavefront w copies row group w's planes and weight row
// tiles 2w, 2w+1; wavefronts 0-3 also copy 64 scales each.  The copies for
// step t + kI8Stages are issued right after the barrier that ends step t,
// into the stage step t used; a wavefront waits for its own copies of step
// t + 1 (vm_wait) before that barrier.
constexpr uint32_t kI8BM = 128;                              // rows of x per workgroup
constexpr uint32_t kI8Stages = 4;
constexpr uint32_t kI8A = (kI8BM / 16) * 2048;               // x planes of one step
constexpr uint32_t kI8B = (kI8TileRows / 16) * 1024;         // weight codes of one step
constexpr uint32_t kI8Stage = kI8A + kI8B + kI8TileRows * 4; // + column scales

// W8 (HT_PATH_W8A8): x is one plane of codes (row group w's at w * 1024 of the
// stage) with a scale per row and K-block (the step's 128 row scales at
// kI8A / 2, copied by wavefronts 4 and 5); per 16 x 16 tile and K-block one
// int8 MFMA, then acc += s * (float(C) * x_scale[row]).
template <bool W8>
__global__ __launch_bounds__(kI8Threads) void gemm_i8_kernel(I8Args a) {
    __shared__ __align__(16) uint8_t lds[kI8Stages * kI8Stage];
    constexpr uint32_t NS = kI8Stages;

    const LayerDev &w = a.w;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wr = wave >> 2, wc = wave & 3;

    uint32_t L = blockIdx.x;
    if ((gridDim.x & 7u) == 0) L = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const uint32_t per_split = a.MT * a.NT;
    const uint32_t zs = L / per_split, rem = L - zs * per_split;
    const uint32_t mt = rem / a.NT, it = rem - mt * a.NT;
    const uint32_t n0 = it * kI8TileRows, m0 = mt * kI8BM;
    const uint32_t KB = w.KB;
    const uint32_t kb0 = zs * a.KBs, kb1 = min(KB, kb0 + a.KBs);
    const uint32_t nsteps = kb1 - kb0;
    if (!int8_tile(w, it, kb0, kb1)) return;   // the whole workgroup; the bfloat16 kernel takes it

    // weight row tile jj of this tile: its first INT8 block of step kb0 and its
    // rows; a tile past the last one borrows the first tile's (valid
    // addresses, outputs not stored)
    const uint32_t *k8 = reinterpret_cast<const uint32_t *>(w.base + w.off_kbidx) + w.nk;
    auto tile_of = [&](uint32_t jj) {
        const uint32_t t = (kI8TileRows / 16) * it + jj;
        return t < w.T ? t : (kI8TileRows / 16) * it;
    };
    const uint32_t tb0 = tile_of(2 * wave), tb1 = tile_of(2 * wave + 1);
    const uint32_t bb0 = k8[tb0 * KB + kb0], nb0 = min(16u, w.N - 16u * tb0);
    const uint32_t bb1 = k8[tb1 * KB + kb0], nb1 = min(16u, w.N - 16u * tb1);
    uint32_t bs = 0, ns = 1;   // scales: wavefronts 0-3, lane -> row tile 4w + l/16
    if (wave < 4) {
        const uint32_t ts = tile_of(4 * wave + (lane >> 4));
        bs = k8[ts * KB + kb0];
        ns = min(16u, w.N - 16u * ts);
    }
    const uint8_t *pay8 = w.base + w.off_pay[1];
    const uint8_t *sc8 = w.base + w.off_scale[1];
    const uint32_t ga = min(m0 / 16 + wave, a.G - 1u);   // this wavefront's row group of x

    // copies of step `step` into stage `st`
    auto issue = [&](uint32_t step, uint32_t st) {
        const uint32_t kb = kb0 + step;
        uint8_t *S = lds + st * kI8Stage;
        if constexpr (W8) {
            lds_copy16(a.q + (uint64_t(ga) * KB + kb) * 1024u + 16u * lane, S + wave * 1024u);
            if (wave == 4 || wave == 5)
                lds_copy4(a.sx + uint64_t(kb) * a.Mp + min(m0 + 64u * (wave - 4u) + lane, a.Mp - 1u),
                          S + kI8A / 2 + (wave - 4u) * 256u);
        } else {
            const uint8_t *qa = a.q + ((uint64_t(ga) * KB + kb) * 2u) * 1024u + 16u * lane;
            lds_copy16(qa, S + wave * 2048u);
            lds_copy16(qa + 1024, S + wave * 2048u + 1024u);
        }
        const uint32_t r = lane & 15u, hq = 16u * (lane >> 4);
        lds_copy16(pay8 + uint64_t(bb0 + step * nb0 + min(r, nb0 - 1u)) * 64u + hq, S + kI8A + (2u * wave) * 1024u);
        lds_copy16(pay8 + uint64_t(bb1 + step * nb1 + min(r, nb1 - 1u)) * 64u + hq,
                   S + kI8A + (2u * wave + 1u) * 1024u);
        if (wave < 4)
            lds_copy4(sc8 + 4u * uint64_t(bs + step * ns + min(r, ns - 1u)), S + kI8A + kI8B + wave * 256u);
    };
    // copies each wavefront issues per step: two planes (W8: one) and two
    // weight row tiles, plus the weight scales for 0-3 (W8: and the x
    // scales for 4-5); wait until those of all but the last `steps` steps
    // issued have landed
    auto wait_steps = [&](int steps) __attribute__((always_inline)) {
        if constexpr (W8) {
            if (wave < 6) {
                if (steps == int(NS - 1)) __builtin_amdgcn_s_waitcnt(vm_wait(int(NS - 1) * 4));
                else __builtin_amdgcn_s_waitcnt(vm_wait(int(NS - 2) * 4));
            } else {
                if (steps == int(NS - 1)) __builtin_amdgcn_s_waitcnt(vm_wait(int(NS - 1) * 3));
                else __builtin_amdgcn_s_waitcnt(vm_wait(int(NS - 2) * 3));
            }
        } else {
            if (wave < 4) {
                if (steps == int(NS - 1)) __builtin_amdgcn_s_waitcnt(vm_wait(int(NS - 1) * 5));
                else __builtin_amdgcn_s_waitcnt(vm_wait(int(NS - 2) * 5));
            } else {
                if (steps == int(NS - 1)) __builtin_amdgcn_s_waitcnt(vm_wait(int(NS - 1) * 4));
                else __builtin_amdgcn_s_waitcnt(vm_wait(int(NS - 2) * 4));
            }
        }
    };
    auto wait_copies = [&](bool keep) {
        if (keep) wait_steps(int(NS - 2));
        else __builtin_amdgcn_s_waitcnt(vm_wait(0));
    };
    // workgroup barrier that leaves outstanding copies in flight
    auto cbar = [&]() {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute8 = [&](uint32_t st) {
        const uint8_t *S = lds + st * kI8Stage;
        i32x4 B[4], A[4];
        float sw[4];
        f32x4 xs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            B[j] = *reinterpret_cast<const i32x4 *>(S + kI8A + (4u * wc + j) * 1024u + 16u * lane);
            sw[j] = *reinterpret_cast<const float *>(S + kI8A + kI8B + 4u * (64u * wc + 16u * j + (lane & 15u)));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            A[i] = *reinterpret_cast<const i32x4 *>(S + (4u * wr + i) * 1024u + 16u * lane);
            xs[i] = *reinterpret_cast<const f32x4 *>(S + kI8A / 2 + 4u * (64u * wr + 16u * i + 4u * (lane >> 4)));
        }
        const i32x4 z = {0, 0, 0, 0};
        i32x4 c[2];
        c[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[0], B[0], z, 0, 0, 0);
#pragma unroll
        for (int k = 1; k <= 16; ++k) {
            if (k < 16) c[k & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[k >> 2], B[k & 3], z, 0, 0, 0);
            const int p = k - 1, b = p & 1;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[p >> 2][p & 3][e] =
                    __builtin_fmaf(sw[p & 3], float(c[b][e]) * xs[p >> 2][e], acc[p >> 2][p & 3][e]);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);   // one tile's fp32 update
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(acc[i][j]));
    };
    auto compute = [&](uint32_t st) {
        const uint8_t *S = lds + st * kI8Stage;
        i32x4 B[4], A[4][2];
        float sw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            B[j] = *reinterpret_cast<const i32x4 *>(S + kI8A + (4u * wc + j) * 1024u + 16u * lane);
            sw[j] = *reinterpret_cast<const float *>(S + kI8A + kI8B + 4u * (64u * wc + 16u * j + (lane & 15u)));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int p = 0; p < 2; ++p)
                A[i][p] = *reinterpret_cast<const i32x4 *>(S + ((4u * wr + i) * 2u + p) * 1024u + 16u * lane);
        // software pipeline over the 16 output tiles: the two MFMAs of tile
        // k+1 are issued before the fp32 update of tile k, so the matrix core
        // and the vector ALU work at the same time
        const i32x4 z = {0, 0, 0, 0};
        i32x4 ch[2], cl[2];
        ch[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[0][0], B[0], z, 0, 0, 0);
        cl[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[0][1], B[0], z, 0, 0, 0);
#pragma unroll
        for (int k = 1; k <= 16; ++k) {
            if (k < 16) {
                ch[k & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[k >> 2][0], B[k & 3], z, 0, 0, 0);
                cl[k & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[k >> 2][1], B[k & 3], z, 0, 0, 0);
            }
            const int p = k - 1, b = p & 1;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[p >> 2][p & 3][e] = __builtin_fmaf(sw[p & 3], float(ch[b][e] * 256 + cl[b][e]), acc[p >> 2][p & 3][e]);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // two MFMAs
            __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);   // one tile's fp32 update
        }
        // keep the updates inside the step (otherwise they sink past the
        // barrier, where both wavefronts of a SIMD would run them together)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(acc[i][j]));
    };

    // prologue: the first NS steps in flight, wait for step 0
#pragma unroll
    for (uint32_t t = 0; t < NS; ++t)
        if (t < nsteps) issue(t, t);
    if (nsteps >= NS) {
        wait_steps(int(NS - 1));
    } else {
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
    }
    cbar();
    uint32_t st = 0;
    for (uint32_t t = 0; t < nsteps; ++t) {
        if constexpr (W8) compute8(st);
        else compute(st);
        if (t + 1 < nsteps) wait_copies(t + NS <= nsteps);
        cbar();
        if (t + NS < nsteps) issue(t + NS, st);
        st = st + 1 == NS ? 0u : st + 1;
    }

    // ---- output: lane holds column l % 16, rows 4 (l / 16) + e of each 16x16 tile ----
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t m = m0 + 64u * wr + 16u * i + 4u * (lane >> 4) + uint32_t(e);
            if (m >= a.M) continue;
            const float rsc = W8 ? 1.0f : a.rs[m];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t n = n0 + 64u * wc + 16u * j + (lane & 15u);
                if (n >= w.N) continue;
                float v = acc[i][j][e] * rsc;
                if (a.partial) {
                    a.partial[(uint64_t(zs) * a.M + m) * w.N + n] = v;
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

struct I8Layout {
    size_t planes, scales, partial, total;   // byte offsets of the regions and total size
};

// planes: whether x is encoded at all; w8: the W8A8 encoding (one plane of
// codes and a scale per row and K-block) instead of the two-plane one
I8Layout i8_layout(const ht_packed_weight *w, int64_t Mt, uint32_t S, bool planes, bool w8) {
    const uint64_t G = uint64_t((Mt + 15) / 16), KB = uint64_t(w->K / kBlockK);
    I8Layout L;
    L.planes = 0;
    L.scales = planes ? align256(G * KB * (w8 ? 1024u : 2048u)) : 0;
    L.partial = L.scales + (planes ? align256((w8 ? KB : 1u) * G * 16u * sizeof(float)) : 0);
    L.total = L.partial + (S > 1 ? size_t(S) * size_t(Mt) * size_t(w->N) * sizeof(float) : 0);
    return L;
}

// What one launch chunk of Mt rows runs, decided on the host from the
// weight's per-format counts:
//   kAll8   every block is INT8: only the int8 kernel, with K-splits of its
//           own when its 128 x 256 tiles are too few to fill the chip;
//   kNone   too few INT8 blocks for any tile to qualify: only the bfloat16
//           MFMA kernel (no encoding of x);
//   kMixed  both kernels over the bfloat16 kernel's K-splits, which then
//           share the partial-sum layout.
enum I8Mode { kAll8, kNone, kMixed };

struct I8Plan {
    I8Mode mode;
    uint32_t S;
};

I8Plan i8_plan(const ht_packed_weight *w, int64_t Mt) {
    const uint64_t KB = uint64_t(w->K / kBlockK);
    const uint64_t NT = uint64_t((w->N + kI8TileRows - 1) / kI8TileRows);
    if (uint64_t(w->counts[1]) == uint64_t(w->N) * KB) {
        const uint64_t tiles = uint64_t((Mt + kI8BM - 1) / kI8BM) * NT;
        uint32_t S = 1;
        if (tiles * 4 < 3 * 256 && KB >= 16) {
            S = uint32_t((256 + tiles - 1) / tiles);
            if (S > KB / 8) S = uint32_t(KB / 8);
            const uint64_t KBs = (KB + S - 1) / S;
            S = uint32_t((KB + KBs - 1) / KBs);
        }
        return {kAll8, S};
    }
    const uint32_t S = gemm_split_count(w, Mt);
    const uint64_t KBs = (KB + S - 1) / S;
    const uint64_t min_rows = uint64_t(w->N) - (NT - 1) * kI8TileRows < kI8TileRows
                                  ? uint64_t(w->N) - (NT - 1) * kI8TileRows : uint64_t(kI8TileRows);
    const uint64_t min_blocks = KB - (S - 1) * KBs;   // the last split's
    if (uint64_t(w->counts[1]) < min_rows * min_blocks) return {kNone, S};
    return {kMixed, S};
}

}  // namespace

bool i8_ok(const ht_packed_weight *w) { return w->row_tile == 16; }

size_t i8_ws(const ht_packed_weight *w, int64_t M, bool w8) {
    const int64_t Mt = M < kI8ChunkRows ? M : kI8ChunkRows;
    const I8Plan P = i8_plan(w, Mt);
    return i8_layout(w, Mt, P.S, P.mode != kNone, w8).total;
}

ht_status run_gemm_i8(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y, uint16_t *ybf,
                      int64_t ldy, int act, void *ws, hipStream_t s, bool w8) {
    uint8_t *wsb = static_cast<uint8_t *>(ws);
    for (int64_t m0 = 0; m0 < M; m0 += kI8ChunkRows) {
        const int64_t Mt = M - m0 < kI8ChunkRows ? M - m0 : kI8ChunkRows;
        const I8Plan P = i8_plan(w, Mt);
        const uint32_t S = P.S;
        const I8Layout Lw = i8_layout(w, Mt, S, P.mode != kNone, w8);
        float *yc = y ? y + m0 * ldy : nullptr;
        uint16_t *ybc = ybf ? ybf + m0 * ldy : nullptr;
        float *part = reinterpret_cast<float *>(wsb + Lw.partial);
        if (P.mode != kNone) {
            const uint32_t G = uint32_t((Mt + 15) / 16);
            I8Args a;
            if (w8) {
                Xq8Args q;
                q.x = x + m0 * ldx;
                q.ldx = ldx;
                q.M = uint32_t(Mt);
                q.KB = uint32_t(w->K / kBlockK);
                q.Mp = 16u * G;
                q.q = wsb + Lw.planes;
                q.sx = reinterpret_cast<float *>(wsb + Lw.scales);
                hipLaunchKernelGGL(xq8_kernel, dim3(uint32_t(Mt)), dim3(256), 0, s, q);
                HT_LAUNCH_CHECK();
                a.q = q.q;
                a.rs = nullptr;
                a.sx = q.sx;
                a.Mp = q.Mp;
            } else {
                XqArgs q;
                q.x = x + m0 * ldx;
                q.ldx = ldx;
                q.M = uint32_t(Mt);
                q.KB = uint32_t(w->K / kBlockK);
                q.q = wsb + Lw.planes;
                q.rs = reinterpret_cast<float *>(wsb + Lw.scales);
                hipLaunchKernelGGL(xq_kernel, dim3(uint32_t(Mt)), dim3(256), 0, s, q);
                HT_LAUNCH_CHECK();
                a.q = q.q;
                a.rs = q.rs;
                a.sx = nullptr;
                a.Mp = 0;
            }
            a.w = layer_dev(w);
            a.y = S > 1 ? nullptr : yc;
            a.ybf = S > 1 ? nullptr : ybc;
            a.partial = S > 1 ? part : nullptr;
            a.ldy = ldy;
            a.M = uint32_t(Mt);
            a.G = G;
            a.KBs = (a.w.KB + S - 1) / S;
            a.MT = uint32_t((Mt + kI8BM - 1) / kI8BM);
            a.NT = uint32_t((a.w.N + kI8TileRows - 1) / kI8TileRows);
            a.act = act;
            if (w8) hipLaunchKernelGGL(gemm_i8_kernel<true>, dim3(a.MT * a.NT * S), dim3(kI8Threads), 0, s, a);
            else hipLaunchKernelGGL(gemm_i8_kernel<false>, dim3(a.MT * a.NT * S), dim3(kI8Threads), 0, s, a);
            HT_LAUNCH_CHECK();
        }
        if (P.mode != kAll8) {
            const ht_status st = gemm_tiles(w, x + m0 * ldx, Mt, ldx, yc, ybc, ldy, act, part, S, P.mode == kMixed, s);
            if (st != HT_OK) return st;
        }
        if (S > 1) {
            const ht_status st = launch_split_reduce(part, S, uint32_t(Mt), uint32_t(w->N), yc, ybc, ldy, act, s);
            if (st != HT_OK) return st;
        }
    }
    return HT_OK;
}

}  // namespace ht
