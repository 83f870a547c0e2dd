// noalloc.hip -- ht_linear_forward_noalloc: ht_linear_forward with its
// workspace in a fixed device array of the library, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// run without an allocator, harnesses that forbid allocation).
//
// The array `scratch` is a file-scope device variable: each GPU the library
// runs on holds its own copy at its own address for the life of the process.
// Host code never passes the array's name to a kernel (on the host it names
// a host-side stand-in); the device address of the current device's copy is
// looked up once per device with hipGetSymbolAddress and kept.  The kernels
// receive that address exactly as they receive a caller's workspace (K-split
// partial sums, and for the int8 path the encoded x), and every byte they
// read from it is written earlier in the same call, so nothing needs
// clearing between calls.  Calls on one GPU share its array: two calls that
// overlap in time on one GPU race.
#include <mutex>

#include "linear_host.h"

static constexpr size_t kScratchBytes = size_t(HT_NOALLOC_SCRATCH_BYTES);

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of each device's copy, once looked up

// The current device's copy of scratch (looked up on the first call on that
// device, with it current).
ht_status scratch_for_current_device(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HT_EHIP;
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HT_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return HT_OK;
}

}  // namespace

extern "C" ht_status ht_linear_forward_noalloc(const ht_packed_weight *w, const uint16_t *x, int64_t M,
                                               int64_t ldx, float *y, int64_t ldy, int32_t act, int32_t path,
                                               ht_stream stream) {
    // descriptor, M and path checks, and the least workspace this call runs
    // with (on HT_PATH_GEMM the two-pass kernel is used when its records fit
    // the array, as ht_linear_forward does given a workspace of this size)
    size_t need = 0;
    ht_status st = ht_linear_workspace(w, M, path, &need);
    if (st != HT_OK) return st;
    if (path == HT_PATH_AUTO) path = ht::auto_linear_path(w, M);
    if (ht::linear_path_ws_min(w, M, path) > kScratchBytes) return HT_ESMALL;
    void *ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != HT_OK) return st;
    // the remaining checks, then the same kernels as ht_linear_forward
    return ht_linear_forward(w, x, M, ldx, y, ldy, act, path, ws, kScratchBytes, stream);
}
