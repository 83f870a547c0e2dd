// int8_tile.h -- which weight tiles the int8 matrix-core path takes, shared by
// that path's kernel (gemm_i8.hip) and the bfloat16 MFMA kernel (gemm.hip),
// which leaves those tiles to it.
#pragma once
#include "gemv_common.h"

namespace ht {

// Weight rows per tile of the int8 matrix-core path (16 row tiles of 16).
constexpr uint32_t kI8TileRows = 256;

// Whether weight rows [256*it, +256) (row tiles 16*it .. 16*it+15) hold only
// INT8 blocks in K-blocks [kb0, kb1): each row tile's INT8 block count over
// the range, read from the kbidx table, equals its rows times the range's
// length.  Row tiles past the last one do not exist and count as INT8.
__device__ __forceinline__ bool int8_tile(const LayerDev &w, uint32_t it, uint32_t kb0, uint32_t kb1) {
    const uint32_t *k8 = reinterpret_cast<const uint32_t *>(w.base + w.off_kbidx) + w.nk;   // INT8's entries
    bool ok = true;
#pragma unroll
    for (uint32_t j = 0; j < kI8TileRows / 16; ++j) {
        const uint32_t t = (kI8TileRows / 16) * it + j;
        if (t < w.T) {
            const uint32_t nr = min(16u, w.N - 16u * t);
            ok = ok && k8[t * w.KB + kb1] - k8[t * w.KB + kb0] == nr * (kb1 - kb0);
        }
    }
    return ok;
}

}  // namespace ht
