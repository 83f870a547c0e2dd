// pack.hip -- compile a format map into execution buffers (HyperTensor 1.0.1
// page, intro: the planner's per-block map is turned into buffers that the
// fused kernels run from; "Key Features": inference-only mode, which drops
// the fp32 master weights -- after packing, the buffers are all the linear
// needs).
//
// Three kernels on the caller's stream:
//   1. count: a workgroup per 256 (row tile t, K-block kb) columns counts,
//      per format, the tile's rows holding that format, scans the counts
//      within its columns into kbidx[f][t*KB + kb], and leaves the
//      segment's totals in the (not yet written) ids area;
//   2. offset: each segment adds the totals of the segments before it (the
//      last also writes each format's total at kbidx[f][T*KB]);
//   3. scatter: one quad of lanes per block, in (t, kb, r) order; a block's
//      position is kbidx[f][t*KB+kb] plus its rank among the column's rows of
//      the same format (wave ballot).  Codes and scales are recomputed from W
//      with the planner's exact arithmetic.  Stores are 16 bytes per lane.
//      Its last workgroup zeroes the alignment padding between regions, so
//      every byte of the buffer is defined.
#include "layout.h"
#include "quant.h"

namespace ht {

struct PackArgs {
    const float *W;
    const uint8_t *fmt;
    uint8_t *buf;
    int64_t ldw;
    uint32_t N, KB, R, lgR, T, nk;   // nk = T*KB + 1
    FastDiv div_kb;
    uint64_t off_kbidx, off_ids[5], off_scale[2], off_pay[5];
    uint32_t counts[5];
};

struct PadArgs {
    uint64_t start[13];
    uint32_t len[13];
    int n;
};

constexpr uint32_t kSeg = 256;   // columns per workgroup of the two index passes

// Index pass 1.  Workgroup s owns columns [256 s, 256 s + 256) (column c =
// t*KB + kb, one per thread): it counts, per format, the rows of tile t
// holding that format in K-block kb, writes the exclusive scan of the counts
// within the segment to kbidx[f][c], and the segment's totals to
// tot[f * S + s].  Counts travel as 16-bit fields, two formats per word (a
// segment holds at most 256 * 16 = 4096 blocks).  Codes above 4 are not
// counted.
__global__ __launch_bounds__(256) void pack_count_kernel(PackArgs a, uint32_t *tot, uint32_t S) {
    __shared__ uint32_t wsum[4][3];
    const uint32_t L = a.T * a.KB;
    const uint32_t c = blockIdx.x * kSeg + threadIdx.x;
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t cc = min(c, L - 1u);
    const uint32_t t = fastdiv(cc, a.div_kb), kb = cc - t * a.KB;
    // all 16 row loads in flight at once (rows past the tile or past N read
    // a valid row and are not counted)
    uint32_t b[16];
#pragma unroll
    for (uint32_t r = 0; r < 16; ++r) b[r] = a.fmt[uint64_t(min(t * a.R + min(r, a.R - 1u), a.N - 1u)) * a.KB + kb];
    uint32_t w[3] = {0u, 0u, 0u};   // formats 0 | 1 << 16, 2 | 3 << 16, 4
#pragma unroll
    for (uint32_t r = 0; r < 16; ++r) {
        const uint32_t f = b[r];
        if (c < L && r < a.R && t * a.R + r < a.N) {
            w[0] += (f == 0u ? 1u : 0u) + (f == 1u ? 0x10000u : 0u);
            w[1] += (f == 2u ? 1u : 0u) + (f == 3u ? 0x10000u : 0u);
            w[2] += f == 4u ? 1u : 0u;
        }
    }
    uint32_t inc[3] = {w[0], w[1], w[2]};   // inclusive scan across the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const uint32_t o = __shfl_up(inc[k], off);
            if (lane >= uint32_t(off)) inc[k] += o;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int k = 0; k < 3; ++k) wsum[wave][k] = inc[k];
    }
    __syncthreads();
    uint32_t ex[3], all[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        uint32_t pre = 0, sum = 0;
#pragma unroll
        for (uint32_t v = 0; v < 4; ++v) {
            pre += v < wave ? wsum[v][k] : 0u;
            sum += wsum[v][k];
        }
        ex[k] = pre + inc[k] - w[k];
        all[k] = sum;
    }
    uint32_t *kbidx = reinterpret_cast<uint32_t *>(a.buf + a.off_kbidx);
    if (c < L) {
#pragma unroll
        for (int f = 0; f < 5; ++f) kbidx[uint64_t(f) * a.nk + c] = (ex[f >> 1] >> (16 * (f & 1))) & 0xFFFFu;
    }
    if (threadIdx.x < 5) {
        const uint32_t f = threadIdx.x;
        const uint32_t v = f == 0 ? all[0] : f == 1 ? all[0] >> 16 : f == 2 ? all[1] : f == 3 ? all[1] >> 16 : all[2];
        tot[f * S + blockIdx.x] = v & 0xFFFFu;
    }
}

// Index pass 2.  Workgroup s adds to its columns' kbidx entries the number of
// format-f blocks in the segments before it (a sum of integers: any order
// gives the same value); the last workgroup also writes each format's total
// at kbidx[f][T*KB].
__global__ __launch_bounds__(256) void pack_offset_kernel(PackArgs a, const uint32_t *tot, uint32_t S) {
    __shared__ uint32_t red[4][5];
    const uint32_t s = blockIdx.x, L = a.T * a.KB;
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t v[5] = {0u, 0u, 0u, 0u, 0u};
    for (uint32_t i = threadIdx.x; i < s; i += kSeg) {
#pragma unroll
        for (int f = 0; f < 5; ++f) v[f] += tot[f * S + i];
    }
#pragma unroll
    for (int f = 0; f < 5; ++f) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v[f] += __shfl_xor(v[f], off);
    }
    if (lane == 0) {
#pragma unroll
        for (int f = 0; f < 5; ++f) red[wave][f] = v[f];
    }
    __syncthreads();
    uint32_t off[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) off[f] = red[0][f] + red[1][f] + red[2][f] + red[3][f];
    uint32_t *kbidx = reinterpret_cast<uint32_t *>(a.buf + a.off_kbidx);
    const uint32_t c = s * kSeg + threadIdx.x;
    if (c < L) {
#pragma unroll
        for (int f = 0; f < 5; ++f) kbidx[uint64_t(f) * a.nk + c] += off[f];
    }
    if (s == S - 1u && threadIdx.x < 5) {
        const uint32_t f = threadIdx.x;
        kbidx[uint64_t(f) * a.nk + L] = (f == 0 ? off[0] : f == 1 ? off[1] : f == 2 ? off[2] : f == 3 ? off[3] : off[4]) +
                                        tot[f * S + s];
    }
}

__global__ __launch_bounds__(256) void pack_scatter_kernel(PackArgs a, PadArgs pad) {
    __shared__ __align__(16) float stage[4][16 * 64];      // per wave: its 16 blocks
    // the last workgroup zeroes the alignment padding between regions (the
    // index passes kept scratch totals in the ids area, so not before now)
    if (blockIdx.x == gridDim.x - 1u) {
        for (int k = 0; k < pad.n; ++k)
            for (uint32_t i = threadIdx.x; i < pad.len[k]; i += 256u) a.buf[pad.start[k] + i] = 0;
    }
    const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
    const uint32_t g = tid >> 2;                 // slot in (t, kb, r) order
    const int part = int(threadIdx.x & 3);
    const uint32_t lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint32_t col = g >> a.lgR;             // t*KB + kb
    const uint32_t r = g & (a.R - 1u);
    const uint32_t t = fastdiv(col, a.div_kb);
    const uint32_t kb = col - t * a.KB;
    const uint32_t n = t * a.R + r;
    const bool valid = col < a.T * a.KB && n < a.N;

    // The wave's 16 blocks (each 256 contiguous bytes of W) as 4 loads of four
    // whole blocks each (16-byte piece p = 64j + lane is piece p % 16 of the
    // wave's block p / 16), through LDS to the compute layout (lane = 4 * block
    // + part holds pieces 4*lane .. 4*lane + 3).  Missing blocks read W's
    // first block and store nothing.
    {
        const uint32_t g0 = (blockIdx.x * 256u + wv * 64u) >> 2;
        f32x4 pc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t p = 64u * j + lane, gg = g0 + (p >> 4);
            const uint32_t cc = gg >> a.lgR, rr = gg & (a.R - 1u);
            const uint32_t tt = fastdiv(cc, a.div_kb), kk = cc - tt * a.KB, nn = tt * a.R + rr;
            const bool ok = cc < a.T * a.KB && nn < a.N;
            pc[j] = ld_stream_f4(a.W + (ok ? int64_t(nn) * a.ldw + kk * 64u : 0) + (p & 15u) * 4u);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4 *>(&stage[wv][(64u * j + lane) * 4u]) = pc[j];
    }
    __syncthreads();
    float w[kPerLane];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(&stage[wv][(4u * lane + k) * 4u]);
        w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
    const uint32_t f = valid ? uint32_t(a.fmt[uint64_t(n) * a.KB + kb]) : 255u;

    // rank among the column's earlier rows with the same format
    uint64_t m[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) m[k] = __ballot(part == 0 && f == uint32_t(k));
    const uint32_t slot = lane >> 2;                     // slot within the wave
    const uint32_t cstart = slot & ~(a.R - 1u);          // first slot of the column (R divides 16)
    const uint64_t before = ((uint64_t(1) << (4 * slot)) - 1u) & ~((uint64_t(1) << (4 * cstart)) - 1u);
    uint64_t mine = 0;
#pragma unroll
    for (int k = 0; k < 5; ++k) mine = (f == uint32_t(k)) ? m[k] : mine;
    const uint32_t rank = uint32_t(__popcll(mine & before));

    if (f > 4u) return;                                  // whole quad leaves together
    const uint32_t *kbidx = reinterpret_cast<const uint32_t *>(a.buf + a.off_kbidx);
    const uint32_t pos = kbidx[uint64_t(f) * a.nk + col] + rank;
    if (pos >= a.counts[f]) return;                      // inconsistent counts: write nothing

    RegionOffsets o;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        o.ids[k] = a.off_ids[k];
        o.pay[k] = a.off_pay[k];
    }
    o.scale[0] = a.off_scale[0];
    o.scale[1] = a.off_scale[1];
    store_block(a.buf, o, f, pos, uint16_t(kb * a.R + r), w, part);
}

}  // namespace ht

using namespace ht;


extern "C" ht_status ht_pack_bytes(int64_t N, int64_t K, int64_t row_tile, const int64_t counts5[5],
                                   size_t *bytes) {
    if (!counts5 || !bytes) return HT_EINVAL;
    Layout L;
    ht_status st = layout_of(N, K, row_tile, counts5, &L);
    if (st != HT_OK) return st;
    *bytes = size_t(L.total);
    return HT_OK;
}

extern "C" ht_status ht_pack(const float *W, int64_t N, int64_t K, int64_t ldw, const uint8_t *fmt_map,
                             int64_t row_tile, const int64_t counts5[5], void *buf, size_t buf_bytes,
                             ht_packed_weight *desc, ht_stream stream) {
    if (!W || !fmt_map || !counts5 || !buf || !desc) return HT_EINVAL;
    if (ldw < K) return HT_ESHAPE;
    Layout L;
    ht_status st = layout_of(N, K, row_tile, counts5, &L);
    if (st != HT_OK) return st;
    if ((reinterpret_cast<uintptr_t>(W) & 15u) || (ldw % 4) || (reinterpret_cast<uintptr_t>(buf) & 255u))
        return HT_EALIGN;
    if (buf_bytes < L.total) return HT_ESMALL;
    const int64_t KB = K / kBlockK;
    const int64_t R = row_tile;
    const int64_t T = (N + R - 1) / R;

    PackArgs a;
    a.W = W;
    a.fmt = fmt_map;
    a.buf = static_cast<uint8_t *>(buf);
    a.ldw = ldw;
    a.N = uint32_t(N);
    a.KB = uint32_t(KB);
    a.R = uint32_t(R);
    a.lgR = uint32_t(__builtin_ctzll(uint64_t(R)));
    a.T = uint32_t(T);
    a.nk = uint32_t(T * KB + 1);
    a.div_kb = make_fastdiv(uint32_t(KB));
    a.off_kbidx = L.kbidx;
    for (int f = 0; f < 5; ++f) { a.off_ids[f] = L.ids[f]; a.off_pay[f] = L.pay[f]; a.counts[f] = uint32_t(counts5[f]); }
    for (int f = 0; f < 2; ++f) a.off_scale[f] = L.scale[f];

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const uint32_t cols = uint32_t(T * KB);
    const uint64_t slots = uint64_t(cols) * uint64_t(R);
    const uint64_t grid = (slots * 4 + 255) / 256;
    if (grid > 0xFFFFFFFFull || slots * 4 > 0xFFFFFFFFull) return HT_ESHAPE;

    PadArgs p;
    const uint64_t starts[12] = {L.kbidx, L.ids[0], L.ids[1], L.ids[2], L.ids[3], L.ids[4],
                                 L.scale[0], L.scale[1], L.pay[0], L.pay[1], L.pay[2], L.pay[3]};
    // region k ends where region k+1 starts; the last (FP32 payload) ends at total
    const uint64_t nexts[12] = {L.ids[0], L.ids[1], L.ids[2], L.ids[3], L.ids[4], L.scale[0],
                                L.scale[1], L.pay[0], L.pay[1], L.pay[2], L.pay[3], L.pay[4]};
    int k = 0;
    for (int i = 0; i < 12; ++i) {
        p.start[k] = starts[i] + L.used[i];
        p.len[k] = uint32_t(nexts[i] - p.start[k]);
        if (p.len[k]) ++k;
    }
    const uint64_t used_last = uint64_t(pay_bytes(4)) * uint64_t(counts5[4]);   // FP32 payload tail
    if (L.total - (L.pay[4] + used_last)) {
        p.start[k] = L.pay[4] + used_last;
        p.len[k] = uint32_t(L.total - p.start[k]);
        ++k;
    }
    p.n = k;
    // the index passes keep 5 * S segment totals in the ids area (at least
    // 2 bytes per column; the scatter rewrites it and zeroes the padding)
    const uint32_t S = uint32_t((uint64_t(cols) + kSeg - 1) / kSeg);
    if (uint64_t(S) * 20u > L.scale[0] - L.ids[0]) return HT_ESHAPE;   // cannot happen (see above)
    uint32_t *tot = reinterpret_cast<uint32_t *>(a.buf + L.ids[0]);
    hipLaunchKernelGGL(pack_count_kernel, dim3(S), dim3(kSeg), 0, s, a, tot, S);
    HT_LAUNCH_CHECK();
    hipLaunchKernelGGL(pack_offset_kernel, dim3(S), dim3(kSeg), 0, s, a, static_cast<const uint32_t *>(tot), S);
    HT_LAUNCH_CHECK();
    hipLaunchKernelGGL(pack_scatter_kernel, dim3(uint32_t(grid)), dim3(256), 0, s, a, p);
    HT_LAUNCH_CHECK();

    desc->N = N;
    desc->K = K;
    desc->row_tile = R;
    desc->n_tiles = T;
    for (int f = 0; f < 5; ++f) {
        desc->counts[f] = counts5[f];
        desc->off_ids[f] = L.ids[f];
        desc->off_payload[f] = L.pay[f];
    }
    desc->off_kbidx = L.kbidx;
    desc->off_scale[0] = L.scale[0];
    desc->off_scale[1] = L.scale[1];
    desc->bytes = L.total;
    desc->layout_version = HT_LAYOUT_VERSION;
    desc->reserved = 0;
    desc->base = buf;
    return HT_OK;
}
