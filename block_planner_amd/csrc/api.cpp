// api.cpp -- host-only parts of the C ABI (no GPU work).
#include "../../include/ht.h"
#include "layout.h"

extern "C" const char *ht_status_string(ht_status s) {
    switch (s) {
    case HT_OK: return "ok";
    case HT_EINVAL: return "invalid argument";
    case HT_ESHAPE: return "invalid shape";
    case HT_EALIGN: return "misaligned pointer or stride";
    case HT_ESMALL: return "buffer or workspace too small";
    case HT_EHIP: return "HIP launch failed";
    }
    return "unknown status";
}

// Defaults: eps_int4 0.08, eps_int8 0.01; eps_bf16 = eps_fp16 = 0 and
// prefer_bf16 = 1 as in the HyperTensor page's "Convert model" call.
extern "C" void ht_plan_params_default(ht_plan_params *p) {
    if (!p) return;
    p->eps_int4 = 0.08;
    p->eps_int8 = 0.01;
    p->eps_bf16 = 0.0;
    p->eps_fp16 = 0.0;
    p->prefer_bf16 = 1;
    p->force_format = -1;
}

namespace ht {

namespace {
constexpr int64_t kPay[5] = {32, 64, 128, 128, 256};   // payload bytes per block: INT4, INT8, BF16, FP16, FP32
uint64_t al256(uint64_t v) { return (v + 255) & ~uint64_t(255); }
}  // namespace

ht_status layout_of(int64_t N, int64_t K, int64_t R, const int64_t c[5], Layout *L) {
    if (N <= 0 || K <= 0 || K % HT_BLOCK_K != 0) return HT_ESHAPE;
    if (!(R == 1 || R == 2 || R == 4 || R == 8 || R == 16)) return HT_ESHAPE;
    const int64_t KB = K / HT_BLOCK_K;
    if (KB * R > 65536) return HT_ESHAPE;                 // block ids are 16-bit (kb * R + r)
    const int64_t T = (N + R - 1) / R;
    if (T * KB + 1 > (int64_t(1) << 31)) return HT_ESHAPE;
    int64_t tot = 0;
    for (int f = 0; f < 5; ++f) {
        if (c[f] < 0 || c[f] > N * KB) return HT_EINVAL;
        tot += c[f];
    }
    if (tot != N * KB) return HT_EINVAL;
    uint64_t o = 0;
    int k = 0;
    L->kbidx = o;
    L->used[k++] = uint64_t(5) * uint64_t(T * KB + 1) * 4u;
    o += al256(L->used[0]);
    for (int f = 0; f < 5; ++f) {
        L->ids[f] = o;
        L->used[k++] = 2u * uint64_t(c[f]);
        o += al256(2u * uint64_t(c[f]));
    }
    for (int f = 0; f < 2; ++f) {
        L->scale[f] = o;
        L->used[k++] = 4u * uint64_t(c[f]);
        o += al256(4u * uint64_t(c[f]));
    }
    for (int f = 0; f < 5; ++f) {
        L->pay[f] = o;
        L->used[k++] = uint64_t(kPay[f]) * uint64_t(c[f]);
        o += al256(uint64_t(kPay[f]) * uint64_t(c[f]));
    }
    L->total = o;
    if (o > 0xFFFFFFFFull) return HT_ESHAPE;   // the kernels address the buffer with 32-bit offsets
    return HT_OK;
}

bool desc_layout_ok(const ht_packed_weight *w) {
    if (!w || w->layout_version != HT_LAYOUT_VERSION) return false;
    const int64_t R = w->row_tile;
    if (w->N <= 0 || w->K <= 0 || w->K % HT_BLOCK_K) return false;
    if (!(R == 1 || R == 2 || R == 4 || R == 8 || R == 16)) return false;
    if (w->n_tiles != (w->N + R - 1) / R) return false;
    Layout L;
    if (layout_of(w->N, w->K, R, w->counts, &L) != HT_OK) return false;
    if (w->off_kbidx != L.kbidx || w->bytes != L.total) return false;
    for (int f = 0; f < 5; ++f)
        if (w->off_ids[f] != L.ids[f] || w->off_payload[f] != L.pay[f]) return false;
    return w->off_scale[0] == L.scale[0] && w->off_scale[1] == L.scale[1];
}

}  // namespace ht

// The block index of a packed buffer in host memory: per format the prefix
// counts start at 0, never decrease and end at the format's count; each
// (tile, K-block) column holds each row of the tile exactly once over the
// five formats, rows ascending within a format, every id naming the column's
// K-block.  Fills the format map this index describes when fmt is given.
extern "C" ht_status ht_check_packed(const ht_packed_weight *w, const void *buf, size_t buf_bytes, uint8_t *fmt) {
    if (!w || !buf || !ht::desc_layout_ok(w)) return HT_EINVAL;
    if (buf_bytes < w->bytes) return HT_ESMALL;
    const uint8_t *b = static_cast<const uint8_t *>(buf);
    const int64_t N = w->N, R = w->row_tile, KB = w->K / HT_BLOCK_K, T = w->n_tiles;
    const int64_t cols = T * KB, nk = cols + 1;
    int lgR = 0;
    while ((int64_t(1) << lgR) < R) ++lgR;
    const uint32_t *kbidx = reinterpret_cast<const uint32_t *>(b + w->off_kbidx);
    for (int f = 0; f < 5; ++f) {
        const uint32_t *k = kbidx + f * nk;
        if (k[0] != 0u || int64_t(k[cols]) != w->counts[f]) return HT_EINVAL;
        for (int64_t c = 0; c < cols; ++c)
            if (k[c + 1] < k[c]) return HT_EINVAL;
    }
    for (int64_t t = 0; t < T; ++t) {
        const int64_t rows = N - t * R < R ? N - t * R : R;
        for (int64_t kb = 0; kb < KB; ++kb) {
            const int64_t c = t * KB + kb;
            uint32_t seen = 0;
            for (int f = 0; f < 5; ++f) {
                const uint16_t *ids = reinterpret_cast<const uint16_t *>(b + w->off_ids[f]);
                int64_t prev = -1;
                for (uint32_t j = kbidx[f * nk + c]; j < kbidx[f * nk + c + 1]; ++j) {
                    const uint32_t id = ids[j], r = id & uint32_t(R - 1);
                    if (int64_t(id >> lgR) != kb || int64_t(r) >= rows || int64_t(r) <= prev) return HT_EINVAL;
                    if (seen & (1u << r)) return HT_EINVAL;
                    seen |= 1u << r;
                    prev = int64_t(r);
                    if (fmt) fmt[(t * R + int64_t(r)) * KB + kb] = uint8_t(f);
                }
            }
            if (seen != (1u << rows) - 1u) return HT_EINVAL;   // rows <= 16
        }
    }
    return HT_OK;
}
