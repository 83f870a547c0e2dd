// gemv_common.h -- pieces of the fused mixed-format GEMV shared by the
// single-layer kernel (linear.hip) and the persistent MLP kernel (mlp.hip).
//
// Work unit: a "chunk" = 64 lanes x 16 bytes of one format's payload, i.e.
// 32 INT4 / 16 INT8 / 8 BF16 / 8 FP16 / 4 FP32 blocks of one row tile, read
// as one coalesced 1 KiB access.  Each lane also reads its block's 16-bit id
// (kb * R + r) and, for integer formats, its fp32 scale.
#pragma once
#include "ht_internal.h"

namespace ht {

// One packed weight as the kernels see it (a copy of the host descriptor's
// fields the device needs).
struct LayerDev {
    const uint8_t *base;
    uint64_t off_kbidx, off_ids[5], off_scale[2], off_pay[5];
    uint32_t counts[5];
    uint32_t N, KB, R, lgR, T, nk;   // nk = T*KB + 1
};

inline LayerDev layer_dev(const ht_packed_weight *w) {
    LayerDev d;
    d.base = static_cast<const uint8_t *>(w->base);
    d.off_kbidx = w->off_kbidx;
    for (int f = 0; f < 5; ++f) {
        d.off_ids[f] = w->off_ids[f];
        d.off_pay[f] = w->off_payload[f];
        d.counts[f] = uint32_t(w->counts[f]);
    }
    d.off_scale[0] = w->off_scale[0];
    d.off_scale[1] = w->off_scale[1];
    d.N = uint32_t(w->N);
    d.KB = uint32_t(w->K / 64);
    d.R = uint32_t(w->row_tile);
    d.lgR = uint32_t(__builtin_ctzll(uint64_t(w->row_tile)));
    d.T = uint32_t(w->n_tiles);
    d.nk = d.T * d.KB + 1;
    return d;
}

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnroll = 8;   // chunks in flight per wave (a 16-row, 4096-wide tile is one batch)


// blocks per chunk and lanes per block, by format
__host__ __device__ constexpr uint32_t bpc_of(int f) { return f == 0 ? 32u : f == 1 ? 16u : f == 4 ? 4u : 8u; }
__device__ constexpr int lpb_of(int f) { return f == 0 ? 2 : f == 1 ? 4 : f == 4 ? 16 : 8; }


__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float fp16_lo(uint32_t v) { return float(__builtin_bit_cast(_Float16, uint16_t(v))); }
__device__ __forceinline__ float fp16_hi(uint32_t v) { return float(__builtin_bit_cast(_Float16, uint16_t(v >> 16))); }
__device__ __forceinline__ float s8(uint32_t v, int b) { return float(int8_t(v >> (8 * b))); }
// signed 4-bit field k (0..7) of v
__device__ __forceinline__ float s4(uint32_t v, int k) { return float(int32_t(v << (28 - 4 * k)) >> 28); }

// Integer formats apply the block's scale after the 64-term partial sum;
// float formats have no scale (the loaded value is then ignored).
template <int F, int M>
__device__ __forceinline__ void store_partial(float *P, uint32_t pstride, uint32_t R, uint32_t r, uint32_t kbl,
                                              const float (&acc)[M], float scale, bool write) {
    if (write) {
#pragma unroll
        for (int m = 0; m < M; ++m) P[(m * R + r) * pstride + kbl] = F < 2 ? acc[m] * scale : acc[m];
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
    store_partial<F, M>(P, pstride, R, r, kbl, acc, scale, ok && part == 0);
}


// Per-lane data of one loaded chunk.
struct Slot {
    uint4 pay;
    float sc;
    uint16_t id;
    int f;     // 0..4, or 5 for "no chunk"
    bool v;    // this lane's block exists
};

// Wave-uniform walk over one tile's chunks in format order (all format-0
// chunks, then format 1, ...): this wave takes global chunk indices first,
// first + step, first + 2*step, ...  The current format's constants are kept
// in scalars and refreshed only when the walk crosses into another format, so
// a chunk costs a handful of scalar instructions.
struct ChunkWalker {
    uint32_t lo[5], hi[5], nch[5], pay[5], ids[5], sc[2];
    const uint8_t *base;
    uint32_t step;
    int f;                       // current format; 5 once the tile is exhausted
    uint32_t ci;                 // chunk index within format f
    // constants of format f (a harmless dummy once f == 5)
    uint32_t c_lo, c_hi, c_nch, c_bpc, c_pb, c_po, c_io, c_so, c_lg;
};

__device__ __forceinline__ void walker_cache(ChunkWalker &w) {
    while (w.f < 5) {   // skip exhausted (or empty) formats
        uint32_t n = 0;
#pragma unroll
        for (int g = 0; g < 5; ++g)
            if (w.f == g) n = w.nch[g];
        if (w.ci < n) break;
        w.ci -= n;
        ++w.f;
    }
    w.c_lo = 0; w.c_hi = 1; w.c_nch = 0xFFFFFFFFu; w.c_bpc = 0; w.c_pb = 0;
    w.c_po = 0; w.c_io = 0; w.c_so = 0; w.c_lg = 4;
#pragma unroll
    for (int g = 0; g < 5; ++g) {
        if (w.f == g) {
            w.c_lo = w.lo[g];
            w.c_hi = w.hi[g];
            w.c_nch = w.nch[g];
            w.c_bpc = bpc_of(g);
            w.c_pb = uint32_t(pay_bytes(g));
            w.c_po = w.pay[g];
            w.c_io = w.ids[g];
            w.c_so = g < 2 ? w.sc[g] : 0u;
            w.c_lg = g == 0 ? 1u : g == 1 ? 2u : g == 4 ? 4u : 3u;
        }
    }
}

__device__ __forceinline__ void walker_start(ChunkWalker &w, uint32_t first, uint32_t step) {
    w.step = step;
    w.f = 0;
    w.ci = first;
    walker_cache(w);
}

__device__ __forceinline__ void walker_advance(ChunkWalker &w) {
    w.ci += w.step;
    if (w.ci >= w.c_nch) walker_cache(w);
}

// Load the walker's current chunk.  Branch-free in the loads: past the end a
// slot reads the first 256 bytes of the buffer, and a lane past the end of
// its format's range re-reads the range's last block; neither lane stores a
// result.  Straight-line loads let the compiler count outstanding loads
// exactly and wait for each chunk's own data only.
__device__ __forceinline__ Slot walker_load(const ChunkWalker &w, uint32_t lane) {
    Slot r;
    uint32_t blk = w.c_lo + w.ci * w.c_bpc + (lane >> w.c_lg);
    r.v = w.f < 5 && blk < w.c_hi;
    blk = min(blk, w.c_hi - 1u);
    const uint32_t sblk = w.f < 2 ? blk : 0u;
    r.f = w.f;
    // the loaded values are used as they are (no arithmetic here), so the
    // wait for each slot's data lands at its first use
    const u32x4 pv = ld_stream_u4(w.base + w.c_po + uint64_t(blk) * w.c_pb + (lane & ((1u << w.c_lg) - 1u)) * 16u);
    r.pay = make_uint4(pv.x, pv.y, pv.z, pv.w);
    r.id = reinterpret_cast<const uint16_t *>(w.base + w.c_io)[blk];
    r.sc = reinterpret_cast<const float *>(w.base + w.c_so)[sblk];   // meaningful for integer formats only
    return r;
}

// A walker over row tile t's blocks in K-blocks [kb0, kb1) of layer w (the
// range of each format's blocks comes from the kbidx table); not started.
__device__ __forceinline__ ChunkWalker chunk_src(const LayerDev &w, uint32_t lo_raw[5], uint32_t hi_raw[5]) {
    ChunkWalker s;
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        s.hi[f] = min(hi_raw[f], w.counts[f]);
        s.lo[f] = min(lo_raw[f], s.hi[f]);
        s.nch[f] = (s.hi[f] - s.lo[f] + bpc_of(f) - 1) / bpc_of(f);
        s.pay[f] = uint32_t(w.off_pay[f]);
        s.ids[f] = uint32_t(w.off_ids[f]);
    }
    s.sc[0] = uint32_t(w.off_scale[0]);
    s.sc[1] = uint32_t(w.off_scale[1]);
    s.base = w.base;
    return s;
}

__device__ __forceinline__ uint32_t n_chunks(const ChunkWalker &s) {
    return s.nch[0] + s.nch[1] + s.nch[2] + s.nch[3] + s.nch[4];
}

// Consume one loaded chunk: dequantise, multiply by x (fp32 in LDS), combine
// the block's lanes and store the block's partial into P[m][r][kb - kb0].
template <int M>
__device__ __forceinline__ void consume(const Slot &sl, uint32_t lane, const float *xs, uint32_t xstride, float *P,
                                        uint32_t pstride, uint32_t kb0, uint32_t nkb, uint32_t R, uint32_t lgR) {
    switch (sl.f) {
    case 0: do_chunk<0, M>(sl.pay, sl.sc, sl.id, sl.v, lane, xs, xstride, P, pstride, kb0, nkb, R, lgR); break;
    case 1: do_chunk<1, M>(sl.pay, sl.sc, sl.id, sl.v, lane, xs, xstride, P, pstride, kb0, nkb, R, lgR); break;
    case 2: do_chunk<2, M>(sl.pay, sl.sc, sl.id, sl.v, lane, xs, xstride, P, pstride, kb0, nkb, R, lgR); break;
    case 3: do_chunk<3, M>(sl.pay, sl.sc, sl.id, sl.v, lane, xs, xstride, P, pstride, kb0, nkb, R, lgR); break;
    case 4: do_chunk<4, M>(sl.pay, sl.sc, sl.id, sl.v, lane, xs, xstride, P, pstride, kb0, nkb, R, lgR); break;
    default: break;
    }
}

// Row sums of P in a fixed order: for (m, r), lane l adds P[m][r][l], then
// P[m][r][l+64], ...; then a fixed butterfly over the 64 lanes.  Calls
// out(m, r, value) on lane 0 for every (m, r) of this wave (rows dealt to the
// workgroup's NW wavefronts in turn).
template <int M, int NW = kWaves, typename Out>
__device__ __forceinline__ void reduce_rows(const float *P, uint32_t pstride, uint32_t R, uint32_t nkb,
                                            uint32_t wave, uint32_t lane, Out out) {
    for (uint32_t pr = wave; pr < M * R; pr += NW) {
        const uint32_t m = pr / R, r = pr - m * R;
        float v = 0.0f;
        for (uint32_t k = lane; k < nkb; k += 64) v += P[(m * R + r) * pstride + k];
        v = group_sum<16>(v);
        v = v + __shfl_xor(v, 16);
        v = v + __shfl_xor(v, 32);
        if (lane == 0) out(m, r, v);
    }
}

}  // namespace ht
