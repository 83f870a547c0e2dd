/*
 * ht.h -- C ABI of the MI355X (gfx950) per-block mixed-precision linear.
 *
 * The method (HyperTensor 1.0.1 project page): a precision planner computes,
 * per weight block, the reconstruction error of each candidate format and
 * keeps the cheapest one within its threshold ("What it does", "Key
 * Features": per-block selection among INT4 / INT8 / FP16 / BF16 / FP32); the
 * resulting map becomes packed buffers that fused kernels multiply from
 * (intro paragraph).  The page's user calls map onto this ABI as follows:
 *   scan_model(...)                    ("Convert model")  -> ht_plan
 *   wrap_model_with_hypertensor(...)   ("Convert model")  -> ht_pack
 *   HyperLinear(...).forward           ("Usage Example")  -> ht_linear_forward
 *   BenchmarkMLP forward (Linear+ReLU) ("Usage Example")  -> ht_mlp_forward
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless marked (host).
 *   - Matrices are row-major; ld* is the row stride in elements.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = the legacy
 *     default stream) and never synchronise, except where stated.
 *   - Every argument check runs on the host before anything is enqueued; a
 *     failed check returns a status and enqueues nothing.  A failed HIP launch
 *     returns HT_EHIP.  Nothing is printed and no exception crosses the ABI.
 *   - The library allocates no device memory: the caller owns W, the format
 *     map, the count array, the packed buffer, x, y and the workspace.
 *   - Device pointers must be 16-byte aligned (HT_EALIGN otherwise), except
 *     the format map and the count array (1 and 8 bytes).
 *   - Calls are re-entrant.  Two calls that share a workspace must not
 *     overlap in time (use one stream, or one workspace per stream).
 *   - A packed-weight descriptor is accepted only when its shape, row tile,
 *     every region offset and its size equal what ht_pack computes from
 *     (N, K, row_tile, counts); otherwise the call returns HT_EINVAL.
 */
#ifndef HT_H
#define HT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HT_BLOCK_K 64          /* K-block width: 64 consecutive entries of a row */
#define HT_LAYOUT_VERSION 1

typedef enum {
    HT_INT4 = 0,  /* symmetric, fp32 scale max|w|/7,   codes in [-7, 7]     */
    HT_INT8 = 1,  /* symmetric, fp32 scale max|w|/127, codes in [-127, 127] */
    HT_BF16 = 2,  /* bfloat16, round to nearest even                        */
    HT_FP16 = 3,  /* IEEE binary16, round to nearest even, subnormals kept  */
    HT_FP32 = 4   /* original fp32 values                                   */
} ht_format;

typedef enum {
    HT_OK = 0,
    HT_EINVAL = 1,  /* NULL pointer, bad eps / force_format / path / act     */
    HT_ESHAPE = 2,  /* N, K or M <= 0, K % 64 != 0, ld < width, layer mismatch,
                       row tile not in {1,2,4,8,16}, (K/64)*row_tile > 65536  */
    HT_EALIGN = 3,  /* a device pointer is not 16-byte aligned               */
    HT_ESMALL = 4,  /* packed buffer or workspace smaller than required      */
    HT_EHIP = 5     /* a HIP launch failed                                   */
} ht_status;

typedef void *ht_stream;    /* hipStream_t */

/* Planner thresholds ("Convert model": eps_fp16 = eps_bf16 = 0.0 and
 * prefer_bf16 = True are the scan's defaults).  A block may take format f when
 * its relative L2 reconstruction error ||w - w_hat|| / ||w|| <= eps_f, tested
 * in squared form in double: err2 <= (eps_f * eps_f) * nrm2, with err2 and
 * nrm2 balanced pairwise sums over the block in natural order.  The block
 * gets the first admissible format of INT4, INT8, then BF16, FP16 (FP16, BF16
 * when prefer_bf16 is 0), then FP32.  A block holding NaN or Inf is FP32. */
typedef struct {
    double eps_int4;       /* default 0.08 */
    double eps_int8;       /* default 0.01 */
    double eps_bf16;       /* default 0.0  */
    double eps_fp16;       /* default 0.0  */
    int32_t prefer_bf16;   /* default 1    */
    int32_t force_format;  /* -1 = plan (default); 0..4 = give every block this format */
} ht_plan_params;

/* Packed execution buffers of one weight W[N, K] (layout version 1).
 * A host-side descriptor filled by ht_pack; valid while the buffer lives.
 * Offsets are in bytes from `base`.  Layout:
 *   R = row_tile, T = ceil(N / R), KB = K / 64.  Blocks are enumerated tile by
 *   tile, K-block by K-block, row by row: (t, kb, r).  Each format keeps its
 *   blocks in that order.  Regions (each 256-byte aligned):
 *     kbidx    uint32 [5][T*KB + 1]: kbidx[f][t*KB + kb] = number of format-f
 *              blocks before (t, kb); entry T*KB is the format's total.
 *     ids_f    uint16 [count_f]: kb * R + r of each block.
 *     scale_f  float  [count_f] for INT4 and INT8: the block's fp32 scale.
 *     pay_f    [count_f][32 | 64 | 128 | 128 | 256 bytes]:
 *              INT4: byte j holds element 32*(j/16) + j%16 in its low nibble
 *                    and that element + 16 in its high nibble (4-bit two's
 *                    complement codes);
 *              INT8: byte i = code i (two's complement);
 *              BF16, FP16: 16-bit patterns in element order;
 *              FP32: the original 32-bit patterns. */
typedef struct {
    int64_t N, K;
    int64_t row_tile;            /* R */
    int64_t n_tiles;             /* T */
    int64_t counts[5];           /* blocks per format */
    uint64_t off_kbidx;
    uint64_t off_ids[5];
    uint64_t off_scale[2];       /* INT4, INT8 */
    uint64_t off_payload[5];
    uint64_t bytes;              /* total size of the packed buffer */
    int32_t layout_version;      /* HT_LAYOUT_VERSION */
    int32_t reserved;
    void *base;                  /* device address of the packed buffer */
} ht_packed_weight;

enum { HT_ACT_NONE = 0, HT_ACT_RELU = 1 };
enum {
    HT_PATH_AUTO = 0,   /* let the library choose                                  */
    HT_PATH_GEMV = 1,   /* one fused GEMV launch per layer                          */
    HT_PATH_FUSED = 2,  /* ht_mlp_forward only: all layers in one persistent launch */
    HT_PATH_GEMM = 3,   /* ht_linear_forward only: LDS dequantisation + bf16 MFMA   */
    HT_PATH_GEMV_MFMA = 4, /* ht_linear_forward only: register dequantisation + bf16 MFMA (row tile 16) */
    HT_PATH_GEMM_I8 = 5,   /* ht_linear_forward only: int8 MFMA for all-INT8 tiles, else as GEMM (row tile 16) */
    HT_PATH_W8A8 = 6       /* ht_linear_forward only: as GEMM_I8 with x as int8 per 64-wide K-block (opt-in W8A8) */
};

/* Human-readable name of a status code (static storage; never NULL). */
const char *ht_status_string(ht_status s);

/* Fill *p with the defaults listed in ht_plan_params. */
void ht_plan_params_default(ht_plan_params *p);

/* ht_plan -- the precision planner ("What it does", "Key Features": per-block
 * selection): each block gets the cheapest format whose error is within its
 * threshold.
 *   W        fp32 [N, ldw], row-major; block (n, kb) = W[n, 64kb .. 64kb+63].
 *   N, K     K % 64 == 0; ldw >= K.
 *   p        (host) thresholds; NULL means the defaults.
 *   fmt_map  uint8 [N, K/64] out: the format code (ht_format) of each block.
 * Integer formats: s = fl32(max|w| / Q) (Q = 7 or 127, correctly rounded
 * fp32 division); q_i = clamp(round_half_even(fl32(w_i / s)), -Q, Q); q = 0
 * when s is 0 or not finite; w_hat_i = q_i * s.  BF16 / FP16: w_hat_i is w_i
 * rounded to nearest even. */
ht_status ht_plan(const float *W, int64_t N, int64_t K, int64_t ldw,
                  const ht_plan_params *p, uint8_t *fmt_map, ht_stream stream);

/* ht_plan_counts -- number of blocks per format in a format map.
 *   counts5  int64 [5] out (device).  The caller copies it to the host to
 *            size the packed buffer (the only host round trip of the path). */
ht_status ht_plan_counts(const uint8_t *fmt_map, int64_t N, int64_t K,
                         int64_t *counts5, ht_stream stream);

/* ht_pack_bytes -- size of the packed buffer (host only, no GPU work).
 *   row_tile in {1, 2, 4, 8, 16}; counts5 (host) from ht_plan_counts.
 *   HT_ESHAPE when the buffer would exceed 4 GiB - 1 (the kernels address
 *   it with 32-bit offsets): split such a weight along N. */
ht_status ht_pack_bytes(int64_t N, int64_t K, int64_t row_tile,
                        const int64_t counts5[5], size_t *bytes);

/* ht_pack -- compile a plan into execution buffers (intro paragraph: the
 * per-block format map is turned into buffers the fused kernels run from).
 *   W, N, K, ldw  as for ht_plan (W is only read; the caller may free it
 *                 afterwards: the buffers hold everything the linear needs,
 *                 the page's inference-only mode).
 *   fmt_map       the plan (any valid codes 0..4 are accepted).
 *   counts5       (host) the plan's per-format counts.
 *   buf           device buffer of buf_bytes >= ht_pack_bytes(...), 256-byte
 *                 aligned; every byte of it is written.
 *   desc          (host) out: the descriptor of the packed weight.
 * Codes and scales are recomputed from W exactly as ht_plan defines them. */
ht_status ht_pack(const float *W, int64_t N, int64_t K, int64_t ldw,
                  const uint8_t *fmt_map, int64_t row_tile, const int64_t counts5[5],
                  void *buf, size_t buf_bytes, ht_packed_weight *desc, ht_stream stream);

/* ht_refresh_bytes -- buffer and workspace sizes for ht_refresh (host only).
 *   buf_bytes   an upper bound of the packed size for any plan of W[N, K]
 *               with this row tile (every split of the blocks into formats);
 *   ws_bytes    the workspace (initialise it once with ht_workspace_init).
 * HT_ESHAPE for the shapes ht_pack refuses. */
ht_status ht_refresh_bytes(int64_t N, int64_t K, int64_t row_tile, size_t *buf_bytes, size_t *ws_bytes);

/* ht_refresh -- re-plan and re-pack W into a buffer allocated in advance, in
 * one pass over W and without a host round trip ("Usage Example":
 * refresh_every, the packed weight following its trained master): the
 * format map, the counts and the packed bytes are exactly those of ht_plan
 * then ht_pack with the same thresholds and row tile.
 *   W, N, K, ldw, p   as ht_plan;  row_tile as ht_pack.
 *   fmt_map   uint8 [N, K/64] out (device): the new plan.
 *   buf       device buffer of buf_bytes, 256-byte aligned; every byte of
 *             the new layout is written (the block index, ids, scales,
 *             payloads and the alignment padding).
 *   counts5   int64 [5] out (device): blocks per format of the new plan.
 *   ws        workspace of ws_bytes >= ht_refresh_bytes(...), initialised
 *             once with ht_workspace_init; each call leaves it ready for the
 *             next.  If a wait between workgroups ever expires (bounded,
 *             about 50 ms), the 32-bit word at byte 8 of ws becomes nonzero
 *             and that call's output is invalid.
 * Then ht_refresh_desc gives the descriptor from the counts (the caller
 * copies the 40 bytes of counts5 to the host).  When the new layout is
 * larger than buf_bytes (a buffer smaller than ht_refresh_bytes's bound)
 * the map and counts are written, the buffer is not, the word at byte 12
 * of ws becomes nonzero and ht_refresh_desc returns HT_ESMALL.
 * W is read once when the weight fits in the registers of the resident
 * workgroups (up to 72 MB of fp32 W on 256 compute units); a larger weight
 * is read twice (the planning pass, then the scatter).  All workgroups of
 * the launch must be resident at once: the grid is sized from the current
 * device's occupancy, and calls that run concurrently on other streams of
 * the same device can delay it (a bounded wait, see ws). */
ht_status ht_refresh(const float *W, int64_t N, int64_t K, int64_t ldw, const ht_plan_params *p,
                     int64_t row_tile, uint8_t *fmt_map, void *buf, size_t buf_bytes, int64_t *counts5,
                     void *ws, size_t ws_bytes, ht_stream stream);

/* ht_refresh_desc -- the descriptor of a buffer ht_refresh filled, from its
 * counts (host only): as ht_pack's descriptor for the same plan.
 * HT_ESMALL when that layout needs more than buf_bytes. */
ht_status ht_refresh_desc(int64_t N, int64_t K, int64_t row_tile, const int64_t counts5[5], void *buf,
                          size_t buf_bytes, ht_packed_weight *desc);

/* ht_check_packed -- validate a packed weight held in HOST memory (e.g. one
 * read from a file) before it is copied to the device and handed to the
 * kernels.  Host only: no GPU work, nothing enqueued.
 *   w        (host) descriptor; w->base is not looked at.
 *   buf      (host) the packed bytes, buf_bytes of them.
 *   fmt      (host, nullable) uint8 [N, K/64] out: the format map the
 *            buffer's block index describes.
 * HT_OK when the descriptor passes the checks every entry point makes (see
 * the conventions above) and the block index is that of a format map: for
 * every format, kbidx starts at 0, never decreases and ends at the format's
 * count; each (tile, K-block) column holds every row of the tile exactly
 * once over the five formats, rows ascending within a format, each id naming
 * that K-block.  HT_EINVAL otherwise; HT_ESMALL when buf_bytes < w->bytes.
 * Payload bytes and scales are not checked (any bytes decode to finite or
 * non-finite values the kernels handle). */
ht_status ht_check_packed(const ht_packed_weight *w, const void *buf, size_t buf_bytes, uint8_t *fmt);

/* ht_linear_workspace -- workspace bytes ht_linear_forward wants for M rows
 * on `path` (HT_PATH_AUTO, HT_PATH_GEMV, HT_PATH_GEMM, HT_PATH_GEMV_MFMA,
 * HT_PATH_GEMM_I8 or HT_PATH_W8A8; HT_EINVAL for HT_PATH_GEMV_MFMA,
 * HT_PATH_GEMM_I8 and HT_PATH_W8A8 with a row tile other than 16).  On
 * HT_PATH_GEMM from 1024 rows this is the two-pass kernel's expanded weight
 * (see ht_linear_forward); less still runs, on the single-pass kernel. */
ht_status ht_linear_workspace(const ht_packed_weight *w, int64_t M, int32_t path,
                              size_t *bytes);

/* ht_linear_forward -- the fused mixed-format linear y = x . W_hat^T
 * ("Key Features": drop-in HyperLinear for nn.Linear, no bias).
 *   w      (host) descriptor from ht_pack.
 *   x      bfloat16 bit patterns [M, ldx], ldx >= K (on HT_PATH_GEMM and
 *          HT_PATH_GEMM_I8 also ldx < 2^28, else HT_ESHAPE).
 *   y      fp32 [M, ldy] out, ldy >= N: y[m, n] = act(sum_k x[m,k] * w_hat[n,k]),
 *          accumulated in fp32; integer blocks apply their scale after the
 *          block's 64-term partial sum.  The result is bitwise reproducible
 *          run to run (fixed-order reductions, no atomics on data).
 *   act    HT_ACT_NONE or HT_ACT_RELU.
 *   path   HT_PATH_GEMV: register dequantisation, 8 rows of x per launch
 *          (for decode, M of a few rows);
 *          HT_PATH_GEMM: blocks dequantised into LDS as bfloat16 (integer
 *          codes exactly; FP16 and FP32 entries as a hi + lo pair, exact for
 *          FP16 and to 16 significant bits for normal FP32 entries, to
 *          2^-133 absolute for fp32 subnormals; an Inf or NaN entry gives
 *          NaN in its output column) and multiplied with bf16 MFMA, fp32
 *          accumulation (for prefill, many rows).  From 1024 rows, when the
 *          256-row x 128-column output tiles number at least 192 and ws holds
 *          ht_linear_workspace's bytes (33 KiB per 128-column x 64-K weight
 *          tile, plus 256 KiB per output tile of a last round that fills at
 *          most half of the compute units: those tiles run as two K halves
 *          whose fp32 sums a second kernel adds, first half then second),
 *          it runs in two passes: the weight tiles are first expanded
 *          once into those bfloat16 planes in ws, which every row tile then
 *          reads; the lo plane's products are added once at the end instead
 *          of per K-block, so the result differs from the single-pass
 *          kernel's (which runs with a smaller workspace) by fp32 rounding;
 *          HT_PATH_GEMV_MFMA: for decode at a few to a few tens of rows
 *          (row tile 16 only, else HT_EINVAL): each block is dequantised
 *          in registers straight into the operands of bf16 MFMAs (the same
 *          bfloat16 planes as HT_PATH_GEMM), 32 rows of x per launch;
 *          HT_PATH_GEMM_I8: for prefill with INT8-heavy plans (row tile 16
 *          only, else HT_EINVAL): a 256-column weight tile (weight rows
 *          [256 i, +256)) whose blocks are all INT8 over the K range of a
 *          split runs on the int8 matrix cores, every other tile exactly as
 *          HT_PATH_GEMM (the same K-splits, unless every block of the
 *          weight is INT8: then the int8 kernel alone, with K-splits of its
 *          own).  The page fixes
 *          no integer encoding of x; here each row m of x is encoded as
 *          x_hat = (256 hi + lo) 2^(E-14) with int8 planes hi, lo,
 *          round-half-even, 2^(E-1) <= max_k |x[m,k]| < 2^E, so
 *          |x_hat - x| <= 2^-14 max_k |x[m,k]|; such a tile computes
 *          x_hat . W_hat^T with exact int32 block sums (a row holding Inf or
 *          NaN gives NaN there).  Range: those tiles add scale * block sum
 *          with the row's 2^(E-14) applied to the finished sum, so their
 *          running sums are 2^(14-E) times the output; an output whose
 *          2^(14-E) sum_k |w_hat[n,k] x_hat[m,k]| reaches FLT_MAX (weights
 *          of magnitude ~1e30 and more) may overflow to Inf or NaN, where
 *          HT_PATH_GEMM would not.  The workspace holds the encoded x
 *          (unless the weight has too few INT8 blocks for any tile, when
 *          the call is HT_PATH_GEMM's); HT_PATH_AUTO never picks this path;
 *          HT_PATH_W8A8: an opt-in mode with int8 activations (W8A8; row
 *          tile 16 only, else HT_EINVAL), the same tiles as HT_PATH_GEMM_I8
 *          but x encoded per token m and 64-wide K-block kb as one int8
 *          code per entry and a power-of-two scale: 2^(E-1) <= max over
 *          the block of |x| < 2^E, q = clamp(rne(x 2^(7-E)), -127, 127),
 *          x_hat = q 2^(E-7), so |x_hat - x| <= 2^-7 of the block maximum
 *          (an all-zero block has x_hat = 0; a block holding Inf or NaN
 *          gives NaN).  Its tiles compute x_hat . W_hat^T with exact int32
 *          block sums, one int8 MFMA per block and the two scales applied
 *          in fp32 per block: a different output function, not within the
 *          bf16 tolerance of the exact linear; other tiles as HT_PATH_GEMM.
 *          HT_PATH_AUTO never picks it;
 *          HT_PATH_AUTO: GEMV_MFMA for 4 <= M <= 32 with row tile 16;
 *          otherwise GEMM when M >= 16, else GEMV.
 *   ws     workspace of ws_bytes >= ht_linear_workspace(w, M, path): K-split
 *          partial sums, added in split order by a second kernel (and on
 *          HT_PATH_GEMM from 1024 rows the expanded weight tiles; there a
 *          workspace that holds only the partials, if any, runs the
 *          single-pass kernel instead). */
ht_status ht_linear_forward(const ht_packed_weight *w, const uint16_t *x, int64_t M,
                            int64_t ldx, float *y, int64_t ldy, int32_t act, int32_t path,
                            void *ws, size_t ws_bytes, ht_stream stream);

/* ht_linear_forward_noalloc -- ht_linear_forward without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that run without an allocator, harnesses
 * that forbid allocation.  The workspace is a fixed array inside the library
 * of HT_NOALLOC_SCRATCH_BYTES on each GPU it runs on, held until the process
 * ends; the call allocates and frees nothing.
 *   Arguments, paths and results as ht_linear_forward (the same kernels:
 *   the result is bitwise that of ht_linear_forward on the same path with a
 *   workspace of HT_NOALLOC_SCRATCH_BYTES; on HT_PATH_GEMM the two-pass
 *   kernel runs when its expanded tiles fit the array, else the single-pass
 *   one).
 *   The current device must be the device of x, y, the packed buffer and
 *   `stream`.
 * HT_ESMALL when the call needs more workspace than the array holds
 * (ht_linear_workspace gives the need; e.g. the int8 path over thousands of
 * rows of a long K).  Every call on a GPU shares that GPU's array, whose
 * contents each call overwrites before reading: calls that overlap in time
 * on one GPU (other streams, other host threads) race, so serialise them. */
#define HT_NOALLOC_SCRATCH_BYTES (32u << 20)
ht_status ht_linear_forward_noalloc(const ht_packed_weight *w, const uint16_t *x, int64_t M,
                                    int64_t ldx, float *y, int64_t ldy, int32_t act, int32_t path,
                                    ht_stream stream);

/* ht_linear_backward_workspace -- workspace bytes ht_linear_backward_data
 * needs for M rows of dY (HT_EINVAL for a row tile other than 16). */
ht_status ht_linear_backward_workspace(const ht_packed_weight *w, int64_t M, size_t *bytes);

/* ht_linear_backward_data -- the input gradient of the linear
 * ("Key Features": training support; "Design Philosophy": custom backward
 * kernels): dX = dY . W_hat over the packed buffers.
 *   w      (host) descriptor from ht_pack; row tile 16 only, else HT_EINVAL.
 *   dy     fp32 [M, lddy], lddy >= N (the gradient of y).
 *   dx     fp32 [M, lddx] out, lddx >= K: dx[m, k] = sum_n dy[m, n] *
 *          w_hat[n, k], summed in a fixed order (bitwise reproducible);
 *          columns k >= K untouched.  Below 16 rows of dY: fp32 arithmetic
 *          on the vector units (integer blocks as (dy * s) * q).  From 16
 *          rows: bf16 MFMAs, dY and w_hat (s * q rounded to fp32 for
 *          integer blocks) each as a hi + lo pair of bfloat16 planes, the
 *          products hi.hi + hi.lo + lo.hi accumulated in fp32 (16
 *          significant bits of each factor; fp32 subnormals kept down to
 *          2^-133; an Inf or NaN weight entry gives NaN in its dx column).
 *   ws     workspace of ws_bytes >= ht_linear_backward_workspace(w, M):
 *          per-split partial sums (over groups of row tiles of W), added
 *          in split order by a second kernel.
 * Forward-only state is not needed: W may have been freed after packing. */
ht_status ht_linear_backward_data(const ht_packed_weight *w, const float *dy, int64_t M, int64_t lddy,
                                  float *dx, int64_t lddx, void *ws, size_t ws_bytes, ht_stream stream);

/* ht_linear_backward_weight -- the gradient for the fp32 master weight under
 * the straight-through estimator ("Design Philosophy": STE for the backward
 * pass; "Key Features": training support): the gradient of W_hat is passed
 * to W unchanged, so dw = dY^T . x.
 *   dy     fp32 [M, lddy], lddy >= N (the gradient of y); M >= 0.
 *   x      bf16 bits [M, ldx], ldx >= K, ldx % 4 == 0: the activations the
 *          forward consumed.
 *   dw     fp32 [N, lddw] out, lddw >= K, lddw % 4 == 0, K % 4 == 0:
 *          dw[n, k] = sum_m dy[m, n] * x[m, k] in a fixed order (bitwise
 *          reproducible); with accumulate != 0 that sum is added to dw
 *          (gradient accumulation); M == 0 writes zeros (or leaves dw).
 *          Below 64 rows: fp32 arithmetic, m in order.  From 64 rows: bf16
 *          MFMAs, dY as a hi + lo pair of bfloat16 planes (16 significant
 *          bits) against the exact bfloat16 x, fp32 accumulation.
 *   No workspace; dy, x and dw 16-byte aligned (HT_EALIGN), 4 * ceil(N / 16)
 *   at most 65535 (HT_ESHAPE).  Needs no packed weight: the plan and the packed
 *   buffers are rebuilt from the updated master by ht_plan / ht_pack. */
ht_status ht_linear_backward_weight(const float *dy, int64_t M, int64_t lddy, const uint16_t *x, int64_t ldx,
                                    int64_t N, int64_t K, float *dw, int64_t lddw, int32_t accumulate,
                                    ht_stream stream);

/* ht_mlp_workspace -- workspace bytes ht_mlp_forward needs for M rows. */
ht_status ht_mlp_workspace(const ht_packed_weight *const *layers, int32_t n_layers,
                           int64_t M, size_t *bytes);

/* ht_workspace_init -- zero-fill a workspace (a fill kernel on `stream`, so it
 * may be captured in a graph).  ht_mlp_forward needs it once per workspace
 * and configuration: the workspace holds a call counter and the tagged
 * activation words of the single-launch path, which every call leaves
 * consistent for the next call with the same layers and M. */
ht_status ht_workspace_init(void *ws, size_t ws_bytes, ht_stream stream);

/* ht_mlp_forward -- the page's BenchmarkMLP ("Usage Example": HyperLinear then
 * ReLU, repeated; no bias):  h_0 = x;  h_l = bf16_rne(relu(h_{l-1} . W_l^T))
 * for l < L;  y = relu(h_{L-1} . W_L^T) in fp32.  Each layer computes exactly
 * what ht_linear_forward computes on the matching path (the same fixed-order
 * sums): the single launch what HT_PATH_GEMV computes, a per-layer launch
 * what its path computes (for HT_PATH_AUTO, the path a single linear of M
 * rows takes).
 *   layers    (host) array of n_layers descriptors; layer l's K must equal
 *             layer l-1's N; hidden widths must be multiples of 8.
 *   x         bfloat16 [M, ldx];  y fp32 [M, ldy] (ldy >= last layer's N).
 *   act_dump  nullable; if set, bfloat16 [n_layers-1][M][N_l] receives every
 *             intermediate h_l (each layer's slab is M * N_l elements, slabs
 *             packed back to back); the layers then read their input from it.
 *   path      HT_PATH_AUTO: one persistent launch for all layers when it fits
 *             (n_layers <= 8, M <= 4, row tile >= 4, x, partial sums and row
 *             buffer within the 160 KiB LDS of a compute unit, the last layer with
 *             no more row tiles than the widest hidden layer, and every
 *             workgroup resident at once), else one launch per layer, each
 *             on the path HT_PATH_AUTO of ht_linear_forward takes for it;
 *             HT_PATH_GEMV: one register-path GEMV launch per layer;
 *             HT_PATH_FUSED: the single launch or HT_EINVAL if it does not fit.
 *   ws        workspace of ws_bytes >= ht_mlp_workspace(...), initialised with
 *             ht_workspace_init before its first use and again whenever it is
 *             used with other layers or another M.  The single launch passes
 *             activations between workgroups through tagged words in it; a
 *             wait for a word is bounded (about 50 ms): if one ever expires,
 *             the 32-bit word at byte offset 8 of ws becomes nonzero and that
 *             call's output is invalid (the launch still terminates).
 * ReLU maps zero, negative values and NaN to +0. */
ht_status ht_mlp_forward(const ht_packed_weight *const *layers, int32_t n_layers,
                         const uint16_t *x, int64_t M, int64_t ldx, float *y, int64_t ldy,
                         uint16_t *act_dump, int32_t path, void *ws, size_t ws_bytes,
                         ht_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* HT_H */
