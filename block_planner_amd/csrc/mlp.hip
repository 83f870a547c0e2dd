// mlp.hip -- the page's BenchmarkMLP forward ("Usage Example": HyperLinear
// layers each followed by ReLU) over packed execution buffers.
//
// Fused path: one persistent launch runs every layer.  Workgroup g owns row
// tile g of each layer (the grid is the largest layer's tile count, and all
// workgroups are resident together).  15 of its 16 wavefronts stream the
// tile's weight chunks: each walks one sequence of chunks across all layers
// (interleaved with the other waves, so every wave gets a mix of formats) in
// groups of two register slots, and refills slot u, as soon as it has been
// consumed, with the chunk one group ahead, possibly the next layer's.  A
// short window keeps each wave's requests flowing steadily; on the measured
// part, deeper windows (4 or 8 slots) streamed more slowly.  The 16th
// wavefront stages the first layer's input and joins the row sums and the
// activation exchange.
//
// Activation exchange without a barrier or cache flushes: a hidden layer's
// outputs are ReLU values, so the sign bit of each bfloat16 is free.  Four
// values are published with one 64-bit atomic store, their four sign bits
// holding a 4-bit call tag.  The workspace keeps a call counter c in 0..14;
// a call's tag is c + 1 (so a zero-initialised word never matches) and the
// next call's counter is (c + 1) mod 15, so two consecutive calls never
// share a tag.  Workgroup 0 advances the counter after gathering every
// hidden layer; the launch is only used when every workgroup owns a row tile
// of some hidden layer, so each has read the counter (its published words
// carry the tag) before the advance.  The activation
// wavefront of every workgroup reads the whole layer with 64-bit atomic
// loads and re-reads any word whose tag is not yet the current one.  Every
// word is written exactly once per call, so a matching tag means the word
// holds this call's values (single-copy atomicity of the 64-bit access).
// All 16 wavefronts take part in reading a layer (one word per lane per
// round for the 4096-wide MLP at batch 1).  The wait is bounded (~50 ms); if
// it ever expires, a flag word in the workspace is set and that call's output
// is invalid, but the launch still terminates.
//
// Per-layer path: one single-layer launch per layer (linear.hip), used when
// the fused launch does not fit (layer count, batch, LDS, residency, tiles).
#include <map>
#include <mutex>
#include <tuple>

#include "gemv_common.h"
#include "linear_host.h"

namespace ht {

constexpr int kMaxLayers = 8;
constexpr int kMaxFusedM = 4;
constexpr uint32_t kSpinLimit = 1u << 21;   // x ~64 clocks per poll: ~50 ms
constexpr uint32_t kSyncBytes = 256;        // [0] call counter, [2] expired-wait flag
constexpr uint32_t kLoadWaves = kWaves - 1; // waves streaming weights; the last one stages the input
constexpr int kSlots = 2;                   // chunks in flight per loading wave
constexpr uint32_t kLdsBudget = 160 * 1024; // LDS of one compute unit

// Phase timestamps, a compile-time variant (built with -DHT_MLP_PHASES, see
// build.py): thread 0 of each workgroup (lane 0 of loading wave 0) records
// the 100 MHz real-time counter at fixed points of a call into
// ht_mlp_phase_ts[workgroup][event]; ht_mlp_phases() copies the table out.
// Events: 0 entry, 1 x staged and block ranges read, 2 wave 0's first two
// chunks consumed; per layer l at 3 + 4l: wave 0 done with its chunks,
// 4 + 4l: all waves done (after the barrier), 5 + 4l: row sums published (or
// the last layer's y written), 6 + 4l: the next layer's x gathered.  In the
// ordinary build the macro is empty.
constexpr int kPhaseEvents = 20;
constexpr int kPhaseGroups = 1024;
#ifdef HT_MLP_PHASES
__device__ uint64_t ht_mlp_phase_ts[kPhaseGroups * kPhaseEvents];
#define HT_PHASE(ev)                                                                                      \
    do {                                                                                                  \
        if (threadIdx.x == 0 && blockIdx.x < kPhaseGroups)                                               \
            ht_mlp_phase_ts[blockIdx.x * kPhaseEvents + (ev)] = __builtin_amdgcn_s_memrealtime();         \
    } while (0)
#else
#define HT_PHASE(ev) \
    do {             \
    } while (0)
#endif

struct MlpArgs {
    LayerDev layer[kMaxLayers];
    uint64_t *hw[kMaxLayers];     // tagged activation words of hidden layer l: [M][N_l / 4]
    uint16_t *hd[kMaxLayers];     // optional plain bfloat16 copy of hidden layer l: [M][N_l]
    const uint16_t *x;
    int64_t ldx;
    float *y;
    int64_t ldy;
    uint32_t *sync;
    uint32_t n_layers;
    uint32_t xcap;                // fp32 entries per row of the x region (max K)
    uint32_t pcap;                // P row stride (max K/64 + 1)
    uint32_t rmax;                // max row tile
};

// Groups of kUnroll chunks this wave walks in a layer with C chunks for its
// tile (at least one, possibly all-empty, so every wave stays in step).
__device__ __forceinline__ uint32_t wave_groups(uint32_t C, uint32_t wave) {
    const uint32_t J = C > wave ? (C - wave + kLoadWaves - 1) / kLoadWaves : 0u;
    const uint32_t g = (J + kSlots - 1) / kSlots;
    return g ? g : 1u;
}

// Chunk loader state for layer l of this workgroup's tile (from the LDS copy
// of the tile's block ranges).
__device__ __forceinline__ ChunkWalker layer_src(const MlpArgs &a, const uint32_t *meta, uint32_t l) {
    uint32_t lo[5], hi[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        lo[f] = __builtin_amdgcn_readfirstlane(meta[l * 10 + f * 2 + 0]);
        hi[f] = __builtin_amdgcn_readfirstlane(meta[l * 10 + f * 2 + 1]);
    }
    return chunk_src(a.layer[l], lo, hi);
}

// Layer 0's input (bfloat16 [M][K], row stride ld) -> LDS fp32 [M][xcap].
template <int M>
__device__ __forceinline__ void stage_input(const uint16_t *x, int64_t ld, uint32_t K, float *xs, uint32_t xstride,
                                            uint32_t lane) {
    const uint32_t per_row = K / 8, total = M * per_row;
    for (uint32_t base = 0; base < total; base += 64 * 8) {
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t i = base + j * 64 + lane;
            if (i < total) {
                const uint32_t m = i / per_row, jj = i - m * per_row;
                v[j] = *reinterpret_cast<const uint4 *>(x + int64_t(m) * ld + jj * 8);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t i = base + j * 64 + lane;
            if (i < total) {
                const uint32_t m = i / per_row, jj = i - m * per_row;
                float4 *d = reinterpret_cast<float4 *>(xs + m * xstride + jj * 8);
                d[0] = make_float4(bf16_lo(v[j].x), bf16_hi(v[j].x), bf16_lo(v[j].y), bf16_hi(v[j].y));
                d[1] = make_float4(bf16_lo(v[j].z), bf16_hi(v[j].z), bf16_lo(v[j].w), bf16_hi(v[j].w));
            }
        }
    }
}

// The tag of a call: bit j of (counter mod 15) + 1 goes to the sign bit of
// value j of every word.  (The counter stays in 0..14; the reduction only
// guards a workspace that was not initialised.)
__device__ __forceinline__ uint64_t tag_bits(uint32_t counter) {
    const uint32_t tag = counter % 15u + 1u;
    return (uint64_t(tag & 1u) << 15) | (uint64_t((tag >> 1) & 1u) << 31) | (uint64_t((tag >> 2) & 1u) << 47) |
           (uint64_t((tag >> 3) & 1u) << 63);
}

// A word is current when its four sign bits spell this call's tag.
__device__ __forceinline__ bool word_ready(uint64_t w, uint64_t tagmask) {
    return (w & 0x8000800080008000ull) == tagmask;
}

// Hidden layer's activations (tagged words [M][N/4]) -> LDS fp32 [M][xcap].
// Wave w reads words w*64 + lane, (w + 16)*64 + lane, ... with 64-bit atomic
// loads and re-reads a word until its tag is current.
template <int M>
__device__ __forceinline__ void gather_hidden(const uint64_t *words, uint32_t N, uint64_t tagmask, float *xs,
                                              uint32_t xstride, uint32_t lane, uint32_t wave, uint32_t *sync) {
    const uint32_t per_row = N / 4, total = M * per_row;
    for (uint32_t i = wave * 64 + lane; i - lane < total; i += kWaves * 64) {   // i - lane is wave-uniform
        uint64_t v = i < total ? __hip_atomic_load(words + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : tagmask;
        uint32_t n = 0;
        while (!__all(word_ready(v, tagmask))) {
            if (++n > kSpinLimit) {
                if (lane == 0) __hip_atomic_store(sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            if (i < total && !word_ready(v, tagmask))
                v = __hip_atomic_load(words + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (i < total) {
            const uint32_t m = i / per_row, q = i - m * per_row;
            const uint64_t w = v & ~0x8000800080008000ull;
            const uint32_t lo = uint32_t(w), hi = uint32_t(w >> 32);
            *reinterpret_cast<float4 *>(xs + m * xstride + q * 4) =
                make_float4(bf16_lo(lo), bf16_hi(lo), bf16_lo(hi), bf16_hi(hi));
        }
    }
}

// Workgroup barrier for LDS data only.  __syncthreads() would also wait
// for every outstanding global load of the wave, i.e. for the next layer's
// chunks the loaders have already requested; none of the barriers below
// orders global memory within the workgroup.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int M>
__global__ __launch_bounds__(kThreads) void mlp_fused_kernel(MlpArgs a) {
    extern __shared__ float lds[];
    uint32_t *meta = reinterpret_cast<uint32_t *>(lds);   // [layer][format][lo, hi]: 80 words
    float *hrow = lds + 128;                              // this tile's row results [M][rmax] (<= 64)
    float *xs = lds + 192;                                // [M][xcap]
    float *P = xs + M * a.xcap;                           // [M][rmax][pcap]
    const uint32_t t = blockIdx.x;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t L = a.n_layers;
    const bool xwave = wave == kLoadWaves;
    // The call counter.  Workgroup 0 advances it after its last gather; the
    // host only runs this launch when every workgroup owns a row tile of some
    // hidden layer (the last layer has no more tiles than the widest hidden
    // one), and every published word carries the tag read here, so by then
    // every workgroup has read the counter.
    HT_PHASE(0);
    const uint32_t epoch =
        __builtin_amdgcn_readfirstlane(__hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const uint64_t tagmask = tag_bits(epoch);

    // block ranges of this tile in every layer -> LDS (10 values per layer)
    if (threadIdx.x < 10 * L) {
        const uint32_t l = threadIdx.x / 10, f = (threadIdx.x % 10) >> 1, end = threadIdx.x & 1;
        const LayerDev &w = a.layer[l];
        uint32_t v = 0;
        if (t < w.T) {
            const uint32_t *kbidx = reinterpret_cast<const uint32_t *>(w.base + w.off_kbidx);
            v = kbidx[uint64_t(f) * w.nk + uint64_t(t) * w.KB + (end ? w.KB : 0u)];
        }
        meta[threadIdx.x] = v;
    }
    if (xwave) stage_input<M>(a.x, a.ldx, a.layer[0].KB * 64, xs, a.xcap, lane);

    // Layer tail, run by every wave: fixed-order row sums, ReLU, then either
    // y (last layer) or this tile's rows published as tagged words.
    auto layer_tail = [&](uint32_t l) {
        const LayerDev &w = a.layer[l];
        const uint32_t R = w.R;
        const bool last = l + 1 == L;
        reduce_rows<M>(P, a.pcap, R, w.KB, wave, lane, [&](uint32_t m, uint32_t r, float v) {
            const uint32_t n = t * R + r;
            v = v > 0.0f ? v : 0.0f;                      // ReLU; +0 for zero, negative and NaN
            if (last) {
                if (n < w.N) a.y[int64_t(m) * a.ldy + n] = v;
            } else {
                hrow[m * R + r] = v;
                if (a.hd[l] && n < w.N) a.hd[l][uint64_t(m) * w.N + n] = f32_to_bf16_rne(v);
            }
        });
        if (last) return;
        lds_barrier();
        // publish: four rows per 64-bit atomic store, the tag in the sign bits
        const uint32_t qpt = R / 4;
        if (threadIdx.x < M * qpt) {
            const uint32_t m = threadIdx.x / qpt, q = threadIdx.x - m * qpt;
            const uint32_t n0 = t * R + 4 * q;
            if (n0 < w.N) {
                const float *h = hrow + m * R + 4 * q;
                const uint64_t word = uint64_t(f32_to_bf16_rne(h[0])) | (uint64_t(f32_to_bf16_rne(h[1])) << 16) |
                                      (uint64_t(f32_to_bf16_rne(h[2])) << 32) |
                                      (uint64_t(f32_to_bf16_rne(h[3])) << 48);
                __hip_atomic_store(a.hw[l] + uint64_t(m) * (w.N / 4) + n0 / 4, word | tagmask, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };

    // The two roles run separate loops with the same sequence of workgroup
    // barriers (per layer: after the chunks, after the row sums, after the
    // next layer's x is in LDS), so their registers never overlap.
    if (xwave) {
        lds_barrier();                        // x staged, block ranges in LDS
        for (uint32_t l = 0; l < L; ++l) {
            lds_barrier();
            layer_tail(l);
            if (l + 1 < L) {
                gather_hidden<M>(a.hw[l], a.layer[l].N, tagmask, xs, a.xcap, lane, wave, a.sync);
                lds_barrier();
            }
        }
    } else {
        // Loader: walk this wave's chunks of every layer in groups of kSlots
        // slots; slot u is refilled right after it is consumed, with the same
        // slot of the next group (possibly the next layer's).
        uint32_t ll = 0, gl = 0;             // layer and group to load next
        // layer 0's block ranges straight from memory (lanes 0..9), so the
        // first weight loads wait for neither the x copy nor the barrier
        ChunkWalker src;
        {
            const LayerDev &w0 = a.layer[0];
            uint32_t v = 0;
            if (lane < 10 && t < w0.T) {
                const uint32_t *kbidx = reinterpret_cast<const uint32_t *>(w0.base + w0.off_kbidx);
                v = kbidx[uint64_t(lane >> 1) * w0.nk + uint64_t(t) * w0.KB + ((lane & 1) ? w0.KB : 0u)];
            }
            uint32_t lo[5], hi[5];
#pragma unroll
            for (int f = 0; f < 5; ++f) {
                lo[f] = __builtin_amdgcn_readlane(v, 2 * f);
                hi[f] = __builtin_amdgcn_readlane(v, 2 * f + 1);
            }
            src = chunk_src(w0, lo, hi);
        }
        walker_start(src, wave, kLoadWaves);
        uint32_t gcount = wave_groups(n_chunks(src), wave);
        auto advance_loader = [&]() {
            if (++gl == gcount) {
                gl = 0;
                if (ll + 1 < L) {
                    ++ll;
                    src = layer_src(a, meta, ll);
                    walker_start(src, wave, kLoadWaves);
                    gcount = wave_groups(n_chunks(src), wave);
                } else {
                    gcount = ~0u;            // past the last layer: every further slot is empty
                    gl = 1u << 24;
                    src.f = 5;
                    walker_cache(src);
                }
            }
        };
        Slot sl[kSlots];
#pragma unroll
        for (int u = 0; u < kSlots; ++u) {
            sl[u] = walker_load(src, lane);
            walker_advance(src);
        }
        lds_barrier();                        // x staged, block ranges of the later layers in LDS
        HT_PHASE(1);
        advance_loader();
        for (uint32_t l = 0; l < L; ++l) {
            const LayerDev &w = a.layer[l];
            const uint32_t KB = w.KB, R = w.R, lgR = w.lgR;
            const uint32_t groups = wave_groups(n_chunks(layer_src(a, meta, l)), wave);
            for (uint32_t g = 0; g < groups; ++g) {
#pragma unroll
                for (int u = 0; u < kSlots; ++u) {
                    consume<M>(sl[u], lane, xs, a.xcap, P, a.pcap, 0u, KB, R, lgR);
                    sl[u] = walker_load(src, lane);
                    walker_advance(src);
                }
                advance_loader();
                if (l == 0 && g == 0) HT_PHASE(2);
            }
            HT_PHASE(3 + 4 * l);
            lds_barrier();
            HT_PHASE(4 + 4 * l);
            layer_tail(l);
            HT_PHASE(5 + 4 * l);
            if (l + 1 < L) {
                gather_hidden<M>(a.hw[l], a.layer[l].N, tagmask, xs, a.xcap, lane, wave, a.sync);
                lds_barrier();
                HT_PHASE(6 + 4 * l);
            }
        }
    }
    if (t == 0 && threadIdx.x == 0)
        __hip_atomic_store(a.sync, (epoch % 15u + 1u) % 15u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t *p, uint64_t n) {
    for (uint64_t i = uint64_t(blockIdx.x) * 256u + threadIdx.x; i < n; i += uint64_t(gridDim.x) * 256u) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

struct MlpPlan {
    size_t part = 0, act = 0;   // bytes: split partials, one activation buffer
    size_t words = 0;           // bytes of tagged activation words (all hidden layers)
    bool fused = false;
    uint32_t grid = 0, lds = 0, xcap = 0, pcap = 0, rmax = 0;
};

// Workgroups of mlp_fused_kernel<M> that can be resident at once on the
// current device with `lds` bytes of LDS each (compute units x occupancy);
// 0 if a query fails.  Probed once per (device, M, LDS bytes): the probe
// (and the LDS attribute the launch needs) costs host calls that would
// otherwise land on every eager decode call.
template <int M>
uint64_t probe_capacity(int dev, uint32_t lds) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&mlp_fused_kernel<M>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsBudget)) != hipSuccess)
        return 0;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&mlp_fused_kernel<M>),
                                                     kThreads, lds) != hipSuccess)
        return 0;
    return uint64_t(per_cu) * uint64_t(cus);
}

bool fused_fits_m(int64_t M, uint32_t grid, uint32_t lds) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    static std::mutex mu;
    static std::map<std::tuple<int, int64_t, uint32_t>, uint64_t> cache;
    const auto key = std::make_tuple(dev, M, lds);
    {
        std::lock_guard<std::mutex> g(mu);
        const auto it = cache.find(key);
        if (it != cache.end()) return it->second >= grid;
    }
    uint64_t cap = 0;
    switch (M) {
    case 1: cap = probe_capacity<1>(dev, lds); break;
    case 2: cap = probe_capacity<2>(dev, lds); break;
    case 3: cap = probe_capacity<3>(dev, lds); break;
    case 4: cap = probe_capacity<4>(dev, lds); break;
    default: return false;
    }
    if (cap) {
        std::lock_guard<std::mutex> g(mu);
        cache[key] = cap;
    }
    return cap >= grid;
}

// Shapes and buffer sizes; `probe_device` also checks residency (a HIP call).
ht_status mlp_plan(const ht_packed_weight *const *layers, int32_t L, int64_t M, bool probe_device, MlpPlan *pl) {
    if (!layers || L <= 0) return HT_EINVAL;
    if (M <= 0) return HT_ESHAPE;
    uint32_t kmax = 0, kbmax = 0, rmax = 0, tmax = 0;
    bool fusable = L <= kMaxLayers && M <= kMaxFusedM;
    for (int32_t l = 0; l < L; ++l) {
        const ht_packed_weight *w = layers[l];
        if (!desc_ok(w)) return HT_EINVAL;
        if (l && w->K != layers[l - 1]->N) return HT_ESHAPE;
        const size_t p = linear_ws(w, M), q = gemm_ws(w, M), r = dec_ok(w) ? dec_ws(w, M) : 0;
        pl->part = p > pl->part ? p : pl->part;
        pl->part = q > pl->part ? q : pl->part;
        pl->part = r > pl->part ? r : pl->part;
        const size_t h = align256(size_t(M) * size_t(w->N) * 2u);
        pl->act = h > pl->act ? h : pl->act;
        if (l + 1 < L) pl->words += align256(size_t(M) * size_t(w->N) * 2u);
        kmax = uint32_t(w->K) > kmax ? uint32_t(w->K) : kmax;
        kbmax = uint32_t(w->K / 64) > kbmax ? uint32_t(w->K / 64) : kbmax;
        rmax = uint32_t(w->row_tile) > rmax ? uint32_t(w->row_tile) : rmax;
        tmax = uint32_t(w->n_tiles) > tmax ? uint32_t(w->n_tiles) : tmax;
        if (w->row_tile < 4) fusable = false;              // four rows per activation word
    }
    if (uint64_t(M) * rmax > 64) fusable = false;           // LDS row buffer
    // every workgroup must own a row tile of some hidden layer: the call
    // counter's advance by workgroup 0 is ordered after their reads of it
    // only through the hidden layers' words
    uint32_t thid = 0;
    for (int32_t l = 0; l + 1 < L; ++l)
        thid = uint32_t(layers[l]->n_tiles) > thid ? uint32_t(layers[l]->n_tiles) : thid;
    if (L > 1 && tmax > thid) fusable = false;
    pl->xcap = kmax;
    pl->pcap = kbmax + 1;
    pl->rmax = rmax;
    pl->grid = tmax;
    pl->lds = 768u + uint32_t(M) * kmax * 4u + uint32_t(M) * rmax * (kbmax + 1u) * 4u;
    if (pl->lds > kLdsBudget) fusable = false;
    pl->fused = fusable && (!probe_device || fused_fits_m(M, pl->grid, pl->lds));
    return HT_OK;
}

size_t mlp_ws_bytes(const MlpPlan &pl) { return kSyncBytes + pl.words + align256(pl.part) + 2 * pl.act; }

template <int M>
void launch_fused(const MlpArgs &a, uint32_t grid, uint32_t lds, hipStream_t s) {
    hipLaunchKernelGGL(mlp_fused_kernel<M>, dim3(grid), dim3(kThreads), lds, s, a);
}

bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace ht

using namespace ht;

extern "C" ht_status ht_mlp_workspace(const ht_packed_weight *const *layers, int32_t n_layers, int64_t M,
                                      size_t *bytes) {
    if (!bytes) return HT_EINVAL;
    MlpPlan pl;
    ht_status st = mlp_plan(layers, n_layers, M, false, &pl);
    if (st != HT_OK) return st;
    *bytes = mlp_ws_bytes(pl);
    return HT_OK;
}

extern "C" ht_status ht_workspace_init(void *ws, size_t ws_bytes, ht_stream stream) {
    if (!ws) return HT_EINVAL;
    if (!al16(ws) || (ws_bytes % 4u)) return HT_EALIGN;
    const uint64_t n = ws_bytes / 4u;
    if (!n) return HT_OK;
    const uint64_t want = (n + 255) / 256;
    const uint32_t grid = uint32_t(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<uint32_t *>(ws), n);
    HT_LAUNCH_CHECK();
    return HT_OK;
}

extern "C" ht_status ht_mlp_forward(const ht_packed_weight *const *layers, int32_t n_layers, const uint16_t *x,
                                    int64_t M, int64_t ldx, float *y, int64_t ldy, uint16_t *act_dump, int32_t path,
                                    void *ws, size_t ws_bytes, ht_stream stream) {
    if (!layers || n_layers <= 0 || !x || !y) return HT_EINVAL;
    if (path != HT_PATH_AUTO && path != HT_PATH_GEMV && path != HT_PATH_FUSED) return HT_EINVAL;
    MlpPlan pl;
    ht_status st = mlp_plan(layers, n_layers, M, false, &pl);
    if (st != HT_OK) return st;
    if (ldx < layers[0]->K || ldy < layers[n_layers - 1]->N) return HT_ESHAPE;
    if (!ws || ws_bytes < mlp_ws_bytes(pl)) return HT_ESMALL;
    if (!al16(x) || !al16(y) || !al16(ws) || (ldx % 8) || (act_dump && !al16(act_dump))) return HT_EALIGN;
    for (int32_t l = 0; l < n_layers; ++l) {
        if (!al16(layers[l]->base)) return HT_EALIGN;
        if (l + 1 < n_layers && (layers[l]->N % 8)) return HT_EALIGN;
    }
    if (path == HT_PATH_FUSED && !pl.fused) return HT_EINVAL;
    bool fused = pl.fused && path != HT_PATH_GEMV;
    if (fused) {
        MlpPlan probe;
        if (mlp_plan(layers, n_layers, M, true, &probe) != HT_OK || !probe.fused) {
            if (path == HT_PATH_FUSED) return HT_EINVAL;
            fused = false;
        }
    }

    uint8_t *wsb = static_cast<uint8_t *>(ws);
    uint8_t *words = wsb + kSyncBytes;
    uint8_t *part = words + pl.words;
    uint16_t *ping[2] = {reinterpret_cast<uint16_t *>(part + align256(pl.part)),
                         reinterpret_cast<uint16_t *>(part + align256(pl.part) + pl.act)};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    if (fused) {
        MlpArgs a;
        size_t woff = 0, dump_off = 0;
        for (int32_t l = 0; l < n_layers; ++l) {
            a.layer[l] = layer_dev(layers[l]);
            a.hw[l] = nullptr;
            a.hd[l] = nullptr;
            if (l + 1 < n_layers) {
                a.hw[l] = reinterpret_cast<uint64_t *>(words + woff);
                woff += align256(size_t(M) * size_t(layers[l]->N) * 2u);
                if (act_dump) a.hd[l] = act_dump + dump_off;
                dump_off += size_t(M) * size_t(layers[l]->N);
            }
        }
        a.x = x;
        a.ldx = ldx;
        a.y = y;
        a.ldy = ldy;
        a.sync = reinterpret_cast<uint32_t *>(wsb);
        a.n_layers = uint32_t(n_layers);
        a.xcap = pl.xcap;
        a.pcap = pl.pcap;
        a.rmax = pl.rmax;
        switch (M) {
        case 1: launch_fused<1>(a, pl.grid, pl.lds, s); break;
        case 2: launch_fused<2>(a, pl.grid, pl.lds, s); break;
        case 3: launch_fused<3>(a, pl.grid, pl.lds, s); break;
        default: launch_fused<4>(a, pl.grid, pl.lds, s); break;
        }
        HT_LAUNCH_CHECK();
        return HT_OK;
    }

    const uint16_t *in = x;
    int64_t ld_in = ldx;
    size_t dump_off = 0;
    // HT_PATH_GEMV: register-path GEMV per layer; HT_PATH_AUTO: each layer on
    // the path a single linear of M rows takes
    for (int32_t l = 0; l < n_layers; ++l) {
        const ht_packed_weight *w = layers[l];
        float *yo = nullptr;
        uint16_t *out = nullptr;
        int64_t ldo = ldy;
        if (l + 1 < n_layers) {
            out = act_dump ? act_dump + dump_off : ping[l & 1];
            dump_off += size_t(M) * size_t(w->N);
            ldo = w->N;
        } else {
            yo = y;
        }
        const int32_t lp = path == HT_PATH_GEMV ? HT_PATH_GEMV : auto_linear_path(w, M);
        st = lp == HT_PATH_GEMM        ? run_gemm(w, in, M, ld_in, yo, out, ldo, HT_ACT_RELU, part, pl.part, s)
             : lp == HT_PATH_GEMV_MFMA ? run_dec(w, in, M, ld_in, yo, out, ldo, HT_ACT_RELU, part, s)
                                       : run_linear(w, in, M, ld_in, yo, out, ldo, HT_ACT_RELU, part, s);
        if (st != HT_OK) return st;
        in = out;
        ld_in = w->N;
    }
    return HT_OK;
}

#ifdef HT_MLP_PHASES
// The phase table of the instrumented build (see HT_PHASE): n words of
// [workgroup][event] timestamps in 10 ns ticks, copied to host memory after
// the work queued so far has finished.
extern "C" ht_status ht_mlp_phases(uint64_t *host_out, size_t n_words) {
    if (!host_out || n_words > size_t(kPhaseGroups) * kPhaseEvents) return HT_EINVAL;
    if (hipDeviceSynchronize() != hipSuccess) return HT_EHIP;
    if (hipMemcpyFromSymbol(host_out, HIP_SYMBOL(ht_mlp_phase_ts), n_words * sizeof(uint64_t)) != hipSuccess)
        return HT_EHIP;
    return HT_OK;
}
#endif
