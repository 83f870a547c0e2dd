// linear_host.h -- host helpers of the single-layer linear, shared with the
// MLP entry points.
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/ht.h"

namespace ht {

// A descriptor the kernels can use: layout version, shape, row tile, and
// every region offset and the size equal to the layout of (N, K, R, counts).
bool desc_ok(const ht_packed_weight *w);

// Workspace bytes of one linear over M rows (the K-split partial sums).
size_t linear_ws(const ht_packed_weight *w, int64_t M);

// Enqueue one linear: y = act(x . W_hat^T), fp32 y or bfloat16 ybf (one of
// them non-null).  Arguments are assumed checked.
ht_status run_linear(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y,
                     uint16_t *ybf, int64_t ldy, int act, void *ws, hipStream_t s);

// Workspace bytes of one linear over M rows on the MFMA path: gemm_ws the
// bytes it prefers (the two-pass kernel's records where it takes M rows),
// gemm_ws_min the least it runs with (the single-pass kernel's K-split
// partials).
size_t gemm_ws(const ht_packed_weight *w, int64_t M);
size_t gemm_ws_min(const ht_packed_weight *w, int64_t M);

// Enqueue one linear on the MFMA path: fp32 y or bfloat16 ybf (one of them
// non-null); the two-pass kernel when it takes M rows and ws_bytes holds its
// records, else the single-pass kernel.  Arguments are assumed checked
// (ws_bytes >= gemm_ws_min).
ht_status run_gemm(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y, uint16_t *ybf,
                   int64_t ldy, int act, void *ws, size_t ws_bytes, hipStream_t s);

// The least workspace ht_linear_forward runs with on `path` (a resolved
// path, not HT_PATH_AUTO); ht_linear_workspace reports the preferred bytes.
size_t linear_path_ws_min(const ht_packed_weight *w, int64_t M, int32_t path);

// The two-pass prefill GEMM (weight tiles expanded once into bfloat16
// planes, then a matrix-core kernel on them): whether the MFMA path takes it
// for M rows (from kXwMinM rows, with enough tiles to fill the chip), its
// workspace bytes (the expanded records), and one linear on it.
constexpr int64_t kXwMinM = 1024;
bool xw_takes(const ht_packed_weight *w, int64_t M);
size_t xw_ws(const ht_packed_weight *w, int64_t M);
ht_status run_gemm_xw(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y, uint16_t *ybf,
                      int64_t ldy, int act, void *ws, hipStream_t s);

// The MFMA path's K-splits for Mt rows (one launch), and its main kernel
// alone over Mt rows: with S > 1 it writes partial[S][Mt][N] (for
// launch_split_reduce), else y or ybf; skip_int8 leaves the column tiles that
// are all INT8 over a split to the int8 matrix-core kernel.
uint32_t gemm_split_count(const ht_packed_weight *w, int64_t Mt);
ht_status gemm_tiles(const ht_packed_weight *w, const uint16_t *x, int64_t Mt, int64_t ldx, float *y, uint16_t *ybf,
                     int64_t ldy, int act, float *partial, uint32_t S, bool skip_int8, hipStream_t s);

// The int8 matrix-core path (row tile 16 only): whether it takes this weight,
// its workspace bytes for M rows (x's int8 planes and row scales, K-split
// partials), and one linear on it (fp32 y or bfloat16 ybf; arguments assumed
// checked).
// With w8 the same path in its W8A8 form (x encoded as one int8 plane with
// a power-of-two scale per row and K-block).
bool i8_ok(const ht_packed_weight *w);
size_t i8_ws(const ht_packed_weight *w, int64_t M, bool w8 = false);
ht_status run_gemm_i8(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y, uint16_t *ybf,
                      int64_t ldy, int act, void *ws, hipStream_t s, bool w8 = false);

// y[m, n] = act(sum over s in order of partial[s][m][n]), fp32 y or bfloat16 ybf.
ht_status launch_split_reduce(const float *partial, uint32_t S, uint32_t M, uint32_t N, float *y, uint16_t *ybf,
                              int64_t ldy, int act, hipStream_t s);

// The register-dequantising MFMA path (row tile 16, packed buffer below 4 GiB,
// its offsets being 32-bit): whether it takes
// this weight, its workspace bytes for M rows (K-split partials), and one
// linear on it (fp32 y or bfloat16 ybf; arguments assumed checked).
bool dec_ok(const ht_packed_weight *w);
size_t dec_ws(const ht_packed_weight *w, int64_t M);
ht_status run_dec(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y, uint16_t *ybf,
                  int64_t ldy, int act, void *ws, hipStream_t s);

// The input gradient dX = dY . W_hat (row tile 16 only): whether it takes
// this weight, its workspace bytes for M rows of dY (per-tile-group sums),
// and one call (arguments assumed checked).
bool bwd_ok(const ht_packed_weight *w);
size_t bwd_ws(const ht_packed_weight *w, int64_t M);
ht_status run_bwd(const ht_packed_weight *w, const float *dy, int64_t M, int64_t lddy, float *dx, int64_t lddx,
                  void *ws, hipStream_t s);

// The input gradient on the matrix cores (row tile 16), for M >= 16 rows of
// dY and a packed buffer below 4 GiB (32-bit buffer offsets): whether it
// takes the call, its workspace bytes (per-split partial tiles) and one call.
constexpr int64_t kBwdGemmMinM = 16;
inline bool bwd_gemm_takes(const ht_packed_weight *w, int64_t M) {
    return M >= kBwdGemmMinM && w->bytes < 0xFFFFFF00ull;
}
size_t bwd_gemm_ws(const ht_packed_weight *w, int64_t M);
ht_status run_bwd_gemm(const ht_packed_weight *w, const float *dy, int64_t M, int64_t lddy, float *dx,
                       int64_t lddx, void *ws, hipStream_t s);

// The weight gradient on the matrix cores, for M >= 64 rows (arguments
// assumed checked).
constexpr int64_t kDwGemmMinM = 64;
ht_status run_dw_gemm(const float *dy, int64_t M, int64_t lddy, const uint16_t *x, int64_t ldx, int64_t N,
                      int64_t K, float *dw, int64_t lddw, int accumulate, hipStream_t s);

// The path HT_PATH_AUTO resolves to for one linear over M rows: the MFMA
// decode path for 4..32 rows (row tile 16, buffer below 4 GiB), otherwise the LDS-staged MFMA path
// from 16 rows and the register path below (1 to 3 rows stay on the register
// path, fastest there; from 4 rows its fp32 copy of x needs a K-split).
inline int32_t auto_linear_path(const ht_packed_weight *w, int64_t M) {
    if (M >= 4 && M <= 32 && dec_ok(w)) return HT_PATH_GEMV_MFMA;
    return M >= 16 ? HT_PATH_GEMM : HT_PATH_GEMV;
}

}  // namespace ht
