// refresh.hip -- re-plan and re-pack a weight in one pass over W (HyperTensor
// 1.0.1 page, "Usage Example": refresh_every, the packed weight following
// its trained master; "Design Philosophy": training-aware).
//
// What ht_plan followed by ht_pack computes, into a buffer allocated in
// advance, with no host round trip in between:
//   1. each workgroup loads its share of W (whole (tile, K-block) columns,
//      64 blocks per sub-round, coalesced through LDS), decides every
//      block's format with the planner's rule, writes the format map and
//      counts each column's blocks per format;
//   2. it publishes its five totals as two tagged 64-bit words and gathers
//      every workgroup's (no fence and no barrier across workgroups: the
//      tag of this call in the words' top 16 bits says they are current;
//      the wait is bounded);
//   3. from the totals of the workgroups before it and of all of them it
//      knows the region offsets of the new layout and every block's
//      position, and writes the block index, ids, scales and payloads
//      exactly as the packer does.
// W is read once when the blocks of every workgroup stay in registers
// between steps 1 and 3 (up to 6 sub-rounds of 16 KiB per workgroup, three
// workgroups per compute unit: 72 MB of fp32 W over 256 compute units); a
// larger weight re-reads W in step 3.  Every
// workgroup must be resident at once (the host sizes the grid for that).
#include <map>
#include <mutex>
#include <tuple>

#include "layout.h"
#include "quant.h"

namespace ht {

constexpr uint32_t kRfThreads = 256;
constexpr uint32_t kRfSub = 64;          // blocks per sub-round (4 lanes each)
constexpr uint32_t kRfHold = 6;          // sub-rounds kept in registers (3 workgroups per compute unit)
constexpr uint32_t kRfMaxJ = 64;         // sub-rounds per workgroup at most
constexpr uint32_t kRfMaxCols = 1024;    // (tile, K-block) columns per workgroup at most
constexpr uint32_t kRfMaxGroups = 2048;  // workgroups at most (two tagged words each)
constexpr uint32_t kRfSync = 256;        // bytes of sync words at the start of the workspace
constexpr uint32_t kRfSpin = 1u << 21;   // x ~64 clocks per poll: ~50 ms
constexpr uint32_t kRfTagCycle = 65535;  // tags 1..65535 in 16 bits

struct RefreshArgs {
    const float *W;
    int64_t ldw;
    uint8_t *fmt;
    uint8_t *buf;
    uint64_t buf_bytes;
    int64_t *counts;                  // out: blocks per format [5]
    uint32_t N, KB, R, lgR, T, nk;    // nk = T*KB + 1
    FastDiv div_kb;
    uint32_t J;                       // sub-rounds per workgroup
    PlanRule rule;
    uint64_t *words;                  // [G][2] tagged per-workgroup totals
    uint32_t *sync;                   // [0] call counter, [2] expired wait, [3] layout larger than the buffer
};

// Load the wave's 16 blocks of sub-round slot range starting at g0 (block
// slots in (tile, K-block, row) order) as 4 fully coalesced 1 KiB loads,
// through LDS, into the compute layout (lane = 4 * block + part holds the
// part's 16 entries).  Slots past the weight read W's first block.
__device__ __forceinline__ void load_blocks(const RefreshArgs &a, uint32_t g0, float *stage, uint32_t lane,
                                            float (&w)[kPerLane]) {
    f32x4 pc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t p = 64u * j + lane, gg = g0 + (p >> 4);
        const uint32_t cc = gg >> a.lgR, rr = gg & (a.R - 1u);
        const uint32_t tt = fastdiv(cc, a.div_kb), kk = cc - tt * a.KB, nn = tt * a.R + rr;
        const bool ok = cc < a.T * a.KB && nn < a.N;
        pc[j] = ld_stream_f4(a.W + (ok ? int64_t(nn) * a.ldw + kk * 64u : 0) + (p & 15u) * 4u);
    }
    // the stage may still be read by this wave's previous sub-round
    __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4 *>(&stage[(64u * j + lane) * 4u]) = pc[j];
    __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(&stage[(4u * lane + k) * 4u]);
        w[4 * k] = v.x;
        w[4 * k + 1] = v.y;
        w[4 * k + 2] = v.z;
        w[4 * k + 3] = v.w;
    }
}

// Per-format masks of the wave's blocks (bit 4s = slot s) and this lane's
// rank among its column's earlier rows of the same format.
__device__ __forceinline__ uint32_t column_rank(uint32_t f, int part, uint32_t lane, uint32_t R, uint64_t (&m)[5]) {
#pragma unroll
    for (int k = 0; k < 5; ++k) m[k] = __ballot(part == 0 && f == uint32_t(k));
    const uint32_t slot = lane >> 2;
    const uint32_t cstart = slot & ~(R - 1u);
    const uint64_t before = ((uint64_t(1) << (4 * slot)) - 1u) & ~((uint64_t(1) << (4 * cstart)) - 1u);
    uint64_t mine = 0;
#pragma unroll
    for (int k = 0; k < 5; ++k) mine = (f == uint32_t(k)) ? m[k] : mine;
    return uint32_t(__popcll(mine & before));
}

// Region offsets of the layout for these totals (as layout_of computes them
// on the host); returns the buffer's total size.
__device__ __forceinline__ uint64_t device_layout(uint32_t nk, const uint32_t (&tot)[5], RegionOffsets &o,
                                                  uint64_t &off_kbidx, uint64_t (&used_end)[13],
                                                  uint64_t (&start)[13]) {
    uint64_t p = 0;
    int k = 0;
    auto region = [&](uint64_t bytes) {
        start[k] = p;
        used_end[k] = p + bytes;
        ++k;
        const uint64_t at = p;
        p += align256(bytes);
        return at;
    };
    off_kbidx = region(5ull * nk * 4u);
#pragma unroll
    for (int f = 0; f < 5; ++f) o.ids[f] = region(2ull * tot[f]);
#pragma unroll
    for (int f = 0; f < 2; ++f) o.scale[f] = region(4ull * tot[f]);
#pragma unroll
    for (int f = 0; f < 5; ++f) o.pay[f] = region(uint64_t(pay_bytes(f)) * tot[f]);
    return p;
}

template <bool EPS16_ZERO, bool HOLD>
__global__ __launch_bounds__(kRfThreads, 3) void refresh_kernel(RefreshArgs a) {
    __shared__ __align__(16) float stage[4][16 * 64];   // per wave: its 16 blocks
    __shared__ uint32_t colc[kRfMaxCols][3];            // per column: counts of formats 0|1<<16, 2|3<<16, 4
    __shared__ uint32_t wsum[4][3];
    __shared__ uint32_t gsum[4][10];
    __shared__ uint32_t pre_s[5], tot_s[5];
    __shared__ uint8_t fl[kRfMaxJ * kRfSub];             // each block's format (255: no block)
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const int part = int(tid & 3u);
    const uint32_t J = a.J;
    const uint32_t cols = J * kRfSub / a.R;               // columns of this workgroup
    const uint32_t col0 = blockIdx.x * cols;              // its first column (t*KB + kb)
    const uint32_t L = a.T * a.KB;

    // ---- 1. plan and count ----------------------------------------------
    float wh[HOLD ? kRfHold : 1][kPerLane];
    auto slot_of = [&](uint32_t j) { return (blockIdx.x * J + j) * kRfSub + (tid >> 2); };
    auto plan_sub = [&](uint32_t j, float (&w)[kPerLane]) {
        const uint32_t g = slot_of(j);
        load_blocks(a, (blockIdx.x * J + j) * kRfSub + wave * 16u, stage[wave], lane, w);
        const uint32_t col = g >> a.lgR, r = g & (a.R - 1u);
        const uint32_t t = fastdiv(min(col, L - 1u), a.div_kb), kb = col - t * a.KB;
        const bool valid = col < L && t * a.R + r < a.N;
        const int fb = block_format<EPS16_ZERO>(w, a.rule);
        const uint32_t f = valid ? uint32_t(fb) : 255u;
        if (part == 0) {
            fl[j * kRfSub + (tid >> 2)] = uint8_t(f);
            if (valid) a.fmt[uint64_t(t * a.R + r) * a.KB + kb] = uint8_t(f);
        }
        uint64_t m[5];
        column_rank(f, part, lane, a.R, m);
        // the first lane of each column in the wave counts it
        const uint32_t slot = lane >> 2;
        if (part == 0 && (slot & (a.R - 1u)) == 0u) {
            const uint64_t cm = ((a.R == 16u ? ~uint64_t(0) : ((uint64_t(1) << (4u * a.R)) - 1u))) << (4u * slot);
            uint32_t c[5];
#pragma unroll
            for (int k = 0; k < 5; ++k) c[k] = uint32_t(__popcll(m[k] & cm));
            const uint32_t cl = (j * kRfSub + wave * 16u + slot) >> a.lgR;
            colc[cl][0] = c[0] | (c[1] << 16);
            colc[cl][1] = c[2] | (c[3] << 16);
            colc[cl][2] = c[4];
        }
    };
    if constexpr (HOLD) {
#pragma unroll
        for (uint32_t j = 0; j < kRfHold; ++j)
            if (j < J) plan_sub(j, wh[j]);
    } else {
        for (uint32_t j = 0; j < J; ++j) plan_sub(j, wh[0]);
    }
    __syncthreads();

    // exclusive prefix of the column counts within the workgroup (each
    // thread scans a run of consecutive columns, then a scan of the runs)
    const uint32_t per = (cols + kRfThreads - 1) / kRfThreads;
    uint32_t run[3] = {0u, 0u, 0u};
    for (uint32_t i = 0; i < per; ++i) {
        const uint32_t c = tid * per + i;
        if (c < cols) {
#pragma unroll
            for (int k = 0; k < 3; ++k) run[k] += colc[c][k];
        }
    }
    uint32_t inc[3] = {run[0], run[1], run[2]};
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
        ex[k] = pre + inc[k] - run[k];
        all[k] = sum;
    }
    __syncthreads();   // every thread has read its run's counts
    for (uint32_t i = 0; i < per; ++i) {
        const uint32_t c = tid * per + i;
        if (c < cols) {
            uint32_t cur[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                cur[k] = colc[c][k];
                colc[c][k] = ex[k];   // now the exclusive prefix of column c
                ex[k] += cur[k];
            }
        }
    }

    // ---- 2. exchange the workgroup totals ---------------------------------
    const uint32_t epoch =
        __builtin_amdgcn_readfirstlane(__hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const uint64_t tag = uint64_t(epoch % kRfTagCycle + 1u) << 48;
    const uint32_t mytot[5] = {all[0] & 0xFFFFu, all[0] >> 16, all[1] & 0xFFFFu, all[1] >> 16, all[2]};
    if (tid == 0) {
        const uint64_t w0 = uint64_t(mytot[0]) | (uint64_t(mytot[1]) << 16) | (uint64_t(mytot[2]) << 32) | tag;
        const uint64_t w1 = uint64_t(mytot[3]) | (uint64_t(mytot[4]) << 16) | tag;
        __hip_atomic_store(a.words + 2u * blockIdx.x, w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.words + 2u * blockIdx.x + 1u, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    uint32_t pre[5] = {0u, 0u, 0u, 0u, 0u}, tot[5] = {0u, 0u, 0u, 0u, 0u};
    const uint32_t nwords = 2u * gridDim.x;
    for (uint32_t i = tid; i - lane < nwords; i += kRfThreads) {   // i - lane is wave-uniform
        uint64_t v = i < nwords ? __hip_atomic_load(a.words + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : tag;
        uint32_t n = 0;
        while (!__all((v & 0xFFFF000000000000ull) == tag)) {
            if (++n > kRfSpin) {
                if (lane == 0) __hip_atomic_store(a.sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            if (i < nwords && (v & 0xFFFF000000000000ull) != tag)
                v = __hip_atomic_load(a.words + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (i < nwords) {
            const uint32_t wg = i >> 1;
            const uint32_t c0 = uint32_t(v) & 0xFFFFu, c1 = uint32_t(v >> 16) & 0xFFFFu, c2 = uint32_t(v >> 32) & 0xFFFFu;
            const bool before = wg < blockIdx.x;
            if ((i & 1u) == 0u) {
                tot[0] += c0; tot[1] += c1; tot[2] += c2;
                if (before) { pre[0] += c0; pre[1] += c1; pre[2] += c2; }
            } else {
                tot[3] += c0; tot[4] += c1;
                if (before) { pre[3] += c0; pre[4] += c1; }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 5; ++k) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            pre[k] += __shfl_xor(pre[k], off);
            tot[k] += __shfl_xor(tot[k], off);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            gsum[wave][k] = pre[k];
            gsum[wave][5 + k] = tot[k];
        }
    }
    __syncthreads();
    if (tid < 5) {
        pre_s[tid] = gsum[0][tid] + gsum[1][tid] + gsum[2][tid] + gsum[3][tid];
        tot_s[tid] = gsum[0][5 + tid] + gsum[1][5 + tid] + gsum[2][5 + tid] + gsum[3][5 + tid];
    }
    __syncthreads();
    uint32_t T5[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) T5[k] = tot_s[k];
    // workgroup 0 has gathered every workgroup's words, each tagged with the
    // counter value its workgroup read: no workgroup reads the counter after
    // this advance
    if (blockIdx.x == 0 && tid == 0) {
        __hip_atomic_store(a.sync, (epoch % kRfTagCycle + 1u) % kRfTagCycle, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        for (int k = 0; k < 5; ++k) a.counts[k] = int64_t(T5[k]);
    }

    // ---- 3. the new layout, the block index and the blocks ----------------
    RegionOffsets o;
    uint64_t off_kbidx, used_end[13], start[13];
    const uint64_t total = device_layout(a.nk, T5, o, off_kbidx, used_end, start);
    if (total > a.buf_bytes) {   // the same decision in every workgroup: write nothing
        if (blockIdx.x == 0 && tid == 0) __hip_atomic_store(a.sync + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    uint32_t *kbidx = reinterpret_cast<uint32_t *>(a.buf + off_kbidx);
    for (uint32_t i = tid; i < cols * 5u; i += kRfThreads) {
        const uint32_t c = i / 5u, f = i - c * 5u;
        if (col0 + c < L) {
            const uint32_t w = colc[c][f >> 1];
            const uint32_t v = f == 4u ? w : ((w >> (16u * (f & 1u))) & 0xFFFFu);
            kbidx[uint64_t(f) * a.nk + col0 + c] = pre_s[f] + v;
        }
    }
    if (blockIdx.x == 0) {
        if (tid < 5) kbidx[uint64_t(tid) * a.nk + L] = tot_s[tid];
        // zero the alignment padding after each region
#pragma unroll
        for (int k = 0; k < 13; ++k) {
            const uint64_t end = k + 1 < 13 ? start[k + 1] : total;
            for (uint64_t i = used_end[k] + tid; i < end; i += kRfThreads) a.buf[i] = 0;
        }
    }
    auto scatter_sub = [&](uint32_t j, uint32_t f, const float (&w)[kPerLane]) {
        uint64_t m[5];
        const uint32_t rank = column_rank(f, part, lane, a.R, m);
        if (f > 4u) return;
        const uint32_t g = slot_of(j);
        const uint32_t col = g >> a.lgR, r = g & (a.R - 1u);
        const uint32_t t = fastdiv(col, a.div_kb), kb = col - t * a.KB;
        const uint32_t cl = col - col0;
        const uint32_t w3 = colc[cl][f >> 1];
        const uint32_t within = f == 4u ? w3 : ((w3 >> (16u * (f & 1u))) & 0xFFFFu);
        const uint32_t pos = pre_s[f] + within + rank;
        if (pos >= tot_s[f]) return;   // totals inconsistent (a wait expired): write nothing out of place
        store_block(a.buf, o, f, pos, uint16_t(kb * a.R + r), w, part);
    };
    if constexpr (HOLD) {
#pragma unroll
        for (uint32_t j = 0; j < kRfHold; ++j)
            if (j < J) scatter_sub(j, fl[j * kRfSub + (tid >> 2)], wh[j]);
    } else {
        for (uint32_t j = 0; j < J; ++j) {
            float w[kPerLane];
            load_blocks(a, (blockIdx.x * J + j) * kRfSub + wave * 16u, stage[wave], lane, w);
            scatter_sub(j, fl[j * kRfSub + (tid >> 2)], w);
        }
    }
}

}  // namespace ht

using namespace ht;

namespace {

// Upper bound of the packed size over every split of the N*K/64 blocks into
// formats: the block index, at most 2 + 4 + 256 bytes per block over the
// ids, scales and payloads, and a 256-byte alignment pad per region.
uint64_t refresh_buf_bound(int64_t N, int64_t K, int64_t R) {
    const uint64_t KB = uint64_t(K / kBlockK), T = uint64_t((N + R - 1) / R), nb = uint64_t(N) * KB;
    return align256(5ull * (T * KB + 1) * 4u) + align256(262ull * nb + 12ull * 256u);
}

uint64_t refresh_ws_bytes() { return kRfSync + 16ull * kRfMaxGroups; }

template <bool E, bool H>
uint64_t rf_capacity_of(int dev) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&refresh_kernel<E, H>),
                                                     kRfThreads, 0) != hipSuccess)
        return 0;
    return uint64_t(per_cu) * uint64_t(cus);
}

// Workgroups of a refresh variant that can be resident at once on the
// current device, probed once per (device, variant).
uint64_t rf_capacity(bool eps16_zero, bool hold) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    static std::mutex mu;
    static std::map<std::tuple<int, bool, bool>, uint64_t> cache;
    const auto key = std::make_tuple(dev, eps16_zero, hold);
    {
        std::lock_guard<std::mutex> g(mu);
        const auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    const uint64_t cap = eps16_zero ? (hold ? rf_capacity_of<true, true>(dev) : rf_capacity_of<true, false>(dev))
                                    : (hold ? rf_capacity_of<false, true>(dev) : rf_capacity_of<false, false>(dev));
    if (cap) {
        std::lock_guard<std::mutex> g(mu);
        cache[key] = cap;
    }
    return cap;
}

ht_status refresh_shape(int64_t N, int64_t K, int64_t R) {
    if (N <= 0 || K <= 0 || K % kBlockK != 0) return HT_ESHAPE;
    if (!(R == 1 || R == 2 || R == 4 || R == 8 || R == 16)) return HT_ESHAPE;
    const int64_t KB = K / kBlockK, T = (N + R - 1) / R;
    if (KB * R > 65536 || T * KB * R > (int64_t(1) << 31)) return HT_ESHAPE;
    if (refresh_buf_bound(N, K, R) > 0xFFFFFFFFull) return HT_ESHAPE;
    return HT_OK;
}

}  // namespace

extern "C" ht_status ht_refresh_bytes(int64_t N, int64_t K, int64_t row_tile, size_t *buf_bytes, size_t *ws_bytes) {
    if (!buf_bytes || !ws_bytes) return HT_EINVAL;
    const ht_status st = refresh_shape(N, K, row_tile);
    if (st != HT_OK) return st;
    *buf_bytes = size_t(refresh_buf_bound(N, K, row_tile));
    *ws_bytes = size_t(refresh_ws_bytes());
    return HT_OK;
}

extern "C" ht_status ht_refresh(const float *W, int64_t N, int64_t K, int64_t ldw, const ht_plan_params *p,
                                int64_t row_tile, uint8_t *fmt_map, void *buf, size_t buf_bytes, int64_t *counts5,
                                void *ws, size_t ws_bytes, ht_stream stream) {
    ht_plan_params def;
    ht_plan_params_default(&def);
    if (!p) p = &def;
    if (!W || !fmt_map || !buf || !counts5 || !ws) return HT_EINVAL;
    ht_status st = refresh_shape(N, K, row_tile);
    if (st != HT_OK) return st;
    if (ldw < K) return HT_ESHAPE;
    if ((reinterpret_cast<uintptr_t>(W) & 15u) || (ldw % 4) || (reinterpret_cast<uintptr_t>(buf) & 255u) ||
        (reinterpret_cast<uintptr_t>(counts5) & 7u) || (reinterpret_cast<uintptr_t>(ws) & 15u))
        return HT_EALIGN;
    const double eps[4] = {p->eps_int4, p->eps_int8, p->eps_bf16, p->eps_fp16};
    for (double e : eps)
        if (!(e >= 0.0) || e > 1e150) return HT_EINVAL;
    if (p->force_format < -1 || p->force_format > 4) return HT_EINVAL;
    if (ws_bytes < refresh_ws_bytes()) return HT_ESMALL;
    const int64_t KB = K / kBlockK, R = row_tile, T = (N + R - 1) / R;
    const uint64_t slots = uint64_t(T * KB * R);
    const bool eps16_zero = p->eps_bf16 == 0.0 && p->eps_fp16 == 0.0;

    // sub-rounds per workgroup: the fewest whose grid is resident at once
    // (a sub-round of 64 blocks always covers whole columns of R <= 16 rows)
    uint32_t J = 1;
    bool hold = false;
    uint64_t G = 0;
    for (;; ++J) {
        if (J > kRfMaxJ || uint64_t(J) * kRfSub / uint64_t(R) > kRfMaxCols) return HT_ESHAPE;
        hold = J <= kRfHold;
        G = (slots + uint64_t(J) * kRfSub - 1) / (uint64_t(J) * kRfSub);
        const uint64_t cap = rf_capacity(eps16_zero, hold);
        if (!cap) return HT_EHIP;
        if (G <= cap && G <= kRfMaxGroups) break;
    }

    RefreshArgs a;
    a.W = W;
    a.ldw = ldw;
    a.fmt = fmt_map;
    a.buf = static_cast<uint8_t *>(buf);
    a.buf_bytes = buf_bytes;
    a.counts = counts5;
    a.N = uint32_t(N);
    a.KB = uint32_t(KB);
    a.R = uint32_t(R);
    a.lgR = uint32_t(__builtin_ctzll(uint64_t(R)));
    a.T = uint32_t(T);
    a.nk = uint32_t(T * KB + 1);
    a.div_kb = make_fastdiv(uint32_t(KB));
    a.J = J;
    for (int i = 0; i < 4; ++i) a.rule.e2[i] = eps[i] * eps[i];
    a.rule.prefer_bf16 = p->prefer_bf16 ? 1 : 0;
    a.rule.force = p->force_format;
    a.sync = static_cast<uint32_t *>(ws);
    a.words = reinterpret_cast<uint64_t *>(static_cast<uint8_t *>(ws) + kRfSync);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<uint32_t>(G)), block(kRfThreads);
    if (eps16_zero) {
        if (hold) hipLaunchKernelGGL((refresh_kernel<true, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((refresh_kernel<true, false>), grid, block, 0, s, a);
    } else {
        if (hold) hipLaunchKernelGGL((refresh_kernel<false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((refresh_kernel<false, false>), grid, block, 0, s, a);
    }
    HT_LAUNCH_CHECK();
    return HT_OK;
}

extern "C" ht_status ht_refresh_desc(int64_t N, int64_t K, int64_t row_tile, const int64_t counts5[5], void *buf,
                                     size_t buf_bytes, ht_packed_weight *desc) {
    if (!counts5 || !buf || !desc) return HT_EINVAL;
    Layout L;
    const ht_status st = layout_of(N, K, row_tile, counts5, &L);
    if (st != HT_OK) return st;
    if (L.total > buf_bytes) return HT_ESMALL;
    desc->N = N;
    desc->K = K;
    desc->row_tile = row_tile;
    desc->n_tiles = (N + row_tile - 1) / row_tile;
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
