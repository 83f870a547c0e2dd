// layout.h -- the packed buffer's region layout (version 1), computed on the
// host from (N, K, row tile, per-format counts).  The packer writes buffers
// in this layout and every entry point that takes a descriptor checks the
// descriptor against it, so the kernels only ever see offsets that lie
// inside the buffer the counts describe.
#pragma once
#include <stdint.h>

#include "../../include/ht.h"

namespace ht {

struct Layout {
    uint64_t kbidx, ids[5], scale[2], pay[5], total;
    uint64_t used[13];   // bytes in use at the start of each region: kbidx, ids x5, scales x2, payloads x5
};

// Regions in order kbidx, ids_f (f = 0..4), scale_f (INT4, INT8), pay_f
// (f = 0..4), each starting at a multiple of 256 bytes.  HT_ESHAPE for a
// shape the kernels cannot address (row tile not in {1,2,4,8,16},
// (K/64)*R > 65536, more than 2^31 columns, more than 4 GiB - 1 bytes);
// HT_EINVAL when a count is negative or the counts do not add up to
// N * K / 64.
ht_status layout_of(int64_t N, int64_t K, int64_t R, const int64_t c[5], Layout *L);

// Layout version, shape, row tile, tile count, and every region offset and
// the size equal to layout_of(N, K, row tile, counts).  The base address is
// not looked at.
bool desc_layout_ok(const ht_packed_weight *w);

}  // namespace ht
