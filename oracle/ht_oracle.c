/*
 * ht_oracle.c -- plain, slow CPU reference of the per-block mixed-precision
 * linear.  TEST INFRASTRUCTURE ONLY: nothing in the library may call it; only
 * the tests, the smoke check and the benchmark's CPU-baseline leg load it.
 *
 * What it follows (HyperTensor 1.0.1 project page):
 *   - "What it does" / "Why HyperTensor?": each weight block is judged on
 *     its own from the error every candidate format would leave, and the
 *     cheapest format within its threshold is kept; the format set is INT4,
 *     INT8, FP16, BF16, FP32 ("Design Philosophy": format-minimal).
 *   - "Key Features": per-block precision selection (PER_BLOCK).
 *   - "Convert model": eps_fp16 = eps_bf16 = 0 and prefer_bf16 = True are the
 *     defaults of the scan.
 *   - Intro paragraph: the planner's map becomes packed buffers that fused
 *     kernels multiply from.
 * The numeric rule used for every block (the pages leave it open and it is
 * fixed by the method's specification):
 *   block      = 64 consecutive entries of one row of W[N, K] (a K-block);
 *   INT4/INT8  = symmetric, fp32 scale s = max|w| / 7 (resp. / 127), codes
 *                q = clamp(round_half_even(w / s), -Q, Q);
 *   BF16/FP16  = round to nearest even of each entry;
 *   admissible = relative L2 error ||w - w_hat|| / ||w|| <= eps_format;
 *   pick       = the first admissible of INT4, INT8, {BF16, FP16} (BF16 first
 *                when prefer_bf16), FP32.
 * Every floating-point step is written out plainly in double precision; the
 * only fp32 operations are the ones the rule itself defines in fp32 (the scale
 * division and the code division).  Compile with -O2 -ffp-contract=off and
 * without fast-math so no fused multiply-add or reassociation creeps in.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BLOCK 64
enum { OR_INT4 = 0, OR_INT8 = 1, OR_BF16 = 2, OR_FP16 = 3, OR_FP32 = 4 };

/* ------------------------------------------------------------------------ */
/* Rounding to the 16-bit formats, written from the IEEE 754 definitions.    */
/* ------------------------------------------------------------------------ */

/* Round a finite value to the nearest number with `mant` fraction bits and
 * minimum normal exponent `emin` (below it, the spacing stays 2^(emin-mant):
 * gradual underflow), ties to even.  Overflow is left to the caller.  All
 * steps are exact in double: a / quantum is a power-of-two scaling and rint()
 * rounds to nearest even under the default rounding mode. */
static double round_to_format(double w, int mant, int emin)
{
    if (w == 0.0) return w;                 /* keeps the sign of zero */
    double a = fabs(w);
    int e;
    frexp(a, &e);                           /* a = f * 2^e, f in [0.5, 1) */
    int ex = e - 1;                         /* floor(log2(a)) */
    if (ex < emin) ex = emin;
    double quantum = ldexp(1.0, ex - mant);
    double r = rint(a / quantum) * quantum;
    return copysign(r, w);
}

/* bfloat16: 7 fraction bits, fp32's exponent range; largest finite value
 * (2 - 2^-7) * 2^127, anything rounding above it becomes infinity. */
double oracle_bf16_round(double w)
{
    if (isnan(w)) return w;
    if (isinf(w)) return w;
    double r = round_to_format(w, 7, -126);
    if (fabs(r) > 0x1.fep127) r = copysign(INFINITY, w);
    return r;
}

/* IEEE binary16: 10 fraction bits, minimum normal exponent -14, largest
 * finite value 65504; anything rounding above it becomes infinity. */
double oracle_fp16_round(double w)
{
    if (isnan(w)) return w;
    if (isinf(w)) return w;
    double r = round_to_format(w, 10, -14);
    if (fabs(r) > 65504.0) r = copysign(INFINITY, w);
    return r;
}

/* Bit pattern of a value already representable in bfloat16 (or +-inf). */
uint16_t oracle_bf16_bits(double r)
{
    float f = (float)r;                     /* exact: bfloat16 is a subset of fp32 */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* Bit pattern of a value already representable in binary16 (or +-inf). */
uint16_t oracle_fp16_bits(double r)
{
    uint16_t s = signbit(r) ? 0x8000u : 0u;
    double a = fabs(r);
    if (isinf(a)) return s | 0x7C00u;
    if (a == 0.0) return s;
    int e;
    frexp(a, &e);
    int ex = e - 1;
    if (ex < -14)                                   /* subnormal: a = m * 2^-24 */
        return s | (uint16_t)(a / ldexp(1.0, -24));
    uint32_t m = (uint32_t)(a / ldexp(1.0, ex - 10)); /* in [1024, 2047] */
    return s | (uint16_t)((ex + 15) << 10) | (uint16_t)(m - 1024u);
}

/* ------------------------------------------------------------------------ */
/* The block rule.                                                           */
/* ------------------------------------------------------------------------ */

/* Balanced pairwise sum in natural order: S[a,b) = S[a,m) + S[m,b), m = (a+b)/2,
 * single-term leaves, in double. */
static double pairwise(const double *t, int a, int b)
{
    if (b - a == 1) return t[a];
    int m = (a + b) / 2;
    return pairwise(t, a, m) + pairwise(t, m, b);
}

static int block_finite(const float *w)
{
    for (int i = 0; i < OR_BLOCK; ++i)
        if (!isfinite(w[i])) return 0;
    return 1;
}

/* Symmetric integer quantisation of one block with Q = 7 (INT4) or 127 (INT8).
 * s = fl32(max|w| / Q); if s is zero or not finite every code is 0; otherwise
 * q_i = clamp(rint(fl32(w_i / s)), -Q, Q).  Writes the fp32 scale and codes. */
void oracle_int_quant_block(const float *w, int Q, float *s_out, int8_t *q)
{
    float amax = 0.0f;
    for (int i = 0; i < OR_BLOCK; ++i) {
        float a = fabsf(w[i]);
        if (isnan(a) || a > amax) amax = a;
        if (isnan(amax)) break;
    }
    float s = amax / (float)Q;                      /* fp32, correctly rounded */
    if (isnan(s)) s = NAN;                          /* one canonical quiet NaN */
    *s_out = s;
    if (s == 0.0f || !isfinite(s)) {
        for (int i = 0; i < OR_BLOCK; ++i) q[i] = 0;
        return;
    }
    for (int i = 0; i < OR_BLOCK; ++i) {
        float t = w[i] / s;                         /* fp32, correctly rounded */
        float r = rintf(t);                         /* round half to even */
        if (r > (float)Q) r = (float)Q;
        if (r < -(float)Q) r = -(float)Q;
        q[i] = (int8_t)r;
    }
}

/* Reconstruction w_hat of one block in format f, in double (exact for every
 * format: q * s has at most 31 significant bits). */
static void dequant_block(const float *w, int f, double *wh)
{
    if (f == OR_INT4 || f == OR_INT8) {
        float s;
        int8_t q[OR_BLOCK];
        oracle_int_quant_block(w, f == OR_INT4 ? 7 : 127, &s, q);
        for (int i = 0; i < OR_BLOCK; ++i) wh[i] = (double)q[i] * (double)s;
    } else if (f == OR_BF16) {
        for (int i = 0; i < OR_BLOCK; ++i) wh[i] = oracle_bf16_round((double)w[i]);
    } else if (f == OR_FP16) {
        for (int i = 0; i < OR_BLOCK; ++i) wh[i] = oracle_fp16_round((double)w[i]);
    } else {
        for (int i = 0; i < OR_BLOCK; ++i) wh[i] = (double)w[i];
    }
}

/* Squared L2 error of format f on one block: pairwise sum of (w - w_hat)^2. */
double oracle_block_err2(const float *w, int f)
{
    double wh[OR_BLOCK], t[OR_BLOCK];
    dequant_block(w, f, wh);
    for (int i = 0; i < OR_BLOCK; ++i) {
        double d = (double)w[i] - wh[i];
        t[i] = d * d;
    }
    return pairwise(t, 0, OR_BLOCK);
}

/* Squared L2 norm of one block: pairwise sum of w^2. */
double oracle_block_nrm2(const float *w)
{
    double t[OR_BLOCK];
    for (int i = 0; i < OR_BLOCK; ++i) t[i] = (double)w[i] * (double)w[i];
    return pairwise(t, 0, OR_BLOCK);
}

/* Relative L2 test in squared form: err2 <= (eps * eps) * nrm2. */
static int admissible(double err2, double eps, double nrm2)
{
    double thr = (eps * eps) * nrm2;
    return err2 <= thr;
}

/* Format of one block.  eps[] is indexed by format (INT4, INT8, BF16, FP16;
 * FP32 has no threshold: its error is zero by definition).  force >= 0 gives
 * every block that format. */
int oracle_pick_block(const float *w, const double *eps, int prefer_bf16, int force)
{
    if (force >= 0) return force;
    if (!block_finite(w)) return OR_FP32;
    double nrm2 = oracle_block_nrm2(w);
    int order[4] = {OR_INT4, OR_INT8, OR_BF16, OR_FP16};
    if (!prefer_bf16) { order[2] = OR_FP16; order[3] = OR_BF16; }
    for (int j = 0; j < 4; ++j) {
        int f = order[j];
        if (admissible(oracle_block_err2(w, f), eps[f], nrm2)) return f;
    }
    return OR_FP32;
}

/* Plan a whole weight: fmt[n * (K/64) + kb] for row n, K-block kb. */
void oracle_plan(const float *W, int64_t N, int64_t K, int64_t ldw,
                 double eps_int4, double eps_int8, double eps_bf16, double eps_fp16,
                 int prefer_bf16, int force, uint8_t *fmt)
{
    double eps[4] = {eps_int4, eps_int8, eps_bf16, eps_fp16};
    int64_t KB = K / OR_BLOCK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t kb = 0; kb < KB; ++kb)
            fmt[n * KB + kb] = (uint8_t)oracle_pick_block(W + n * ldw + kb * OR_BLOCK,
                                                          eps, prefer_bf16, force);
}

/* Per-block errors for inspection: err2[(n*KB+kb)*5 + f] and nrm2[n*KB+kb]. */
void oracle_block_errors(const float *W, int64_t N, int64_t K, int64_t ldw,
                         double *err2, double *nrm2)
{
    int64_t KB = K / OR_BLOCK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t kb = 0; kb < KB; ++kb) {
            const float *w = W + n * ldw + kb * OR_BLOCK;
            int64_t b = n * KB + kb;
            for (int f = 0; f < 5; ++f) err2[b * 5 + f] = oracle_block_err2(w, f);
            nrm2[b] = oracle_block_nrm2(w);
        }
}

/* Scales and codes of every block for one integer format (Q = 7 or 127),
 * whatever the plan chose: scale[n*KB+kb], codes[n*K + k]. */
void oracle_int_quant(const float *W, int64_t N, int64_t K, int64_t ldw, int Q,
                      float *scale, int8_t *codes)
{
    int64_t KB = K / OR_BLOCK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t kb = 0; kb < KB; ++kb)
            oracle_int_quant_block(W + n * ldw + kb * OR_BLOCK, Q, &scale[n * KB + kb],
                                   codes + n * K + kb * OR_BLOCK);
}

/* Dequantised weight W_hat[n*K + k] (double) under a plan. */
void oracle_dequant(const float *W, int64_t N, int64_t K, int64_t ldw,
                    const uint8_t *fmt, double *What)
{
    int64_t KB = K / OR_BLOCK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t kb = 0; kb < KB; ++kb)
            dequant_block(W + n * ldw + kb * OR_BLOCK, fmt[n * KB + kb],
                          What + n * K + kb * OR_BLOCK);
}

/* ------------------------------------------------------------------------ */
/* The linear: y[m, n] = sum_k x[m, k] * w_hat[n, k], in double.             */
/* x is bfloat16 (bit patterns), widened exactly.                            */
/* ------------------------------------------------------------------------ */
static double bf16_widen(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

void oracle_linear(const float *W, int64_t N, int64_t K, int64_t ldw, const uint8_t *fmt,
                   const uint16_t *x, int64_t M, int64_t ldx, double *y, int64_t ldy)
{
    int64_t KB = K / OR_BLOCK;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K));
    double *wrow = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) xd[m * K + k] = bf16_widen(x[m * ldx + k]);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t kb = 0; kb < KB; ++kb)
            dequant_block(W + n * ldw + kb * OR_BLOCK, fmt[n * KB + kb], wrow + kb * OR_BLOCK);
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xd[m * K + k] * wrow[k];
            y[m * ldy + n] = acc;
        }
    }
    free(wrow);
    free(xd);
}

/* Selected outputs only: y_s = sum_k x[m_s, k] * w_hat[n_s, k] for S pairs. */
void oracle_linear_sampled(const float *W, int64_t K, int64_t ldw, const uint8_t *fmt,
                           const uint16_t *x, int64_t ldx, const int64_t *m_idx,
                           const int64_t *n_idx, int64_t S, double *y)
{
    int64_t KB = K / OR_BLOCK;
    double wh[OR_BLOCK];
    for (int64_t s = 0; s < S; ++s) {
        int64_t m = m_idx[s], n = n_idx[s];
        double acc = 0.0;
        for (int64_t kb = 0; kb < KB; ++kb) {
            dequant_block(W + n * ldw + kb * OR_BLOCK, fmt[n * KB + kb], wh);
            for (int i = 0; i < OR_BLOCK; ++i)
                acc += bf16_widen(x[m * ldx + kb * OR_BLOCK + i]) * wh[i];
        }
        y[s] = acc;
    }
}

/* ReLU in double, the last MLP layer's output (the page's BenchmarkMLP is
 * Linear + ReLU, repeated): z where z > 0, else +0, so zero (of either
 * sign), negative values and NaN all give +0.  The page does not say what
 * ReLU does with NaN; this is the reading used for every layer. */
void oracle_relu(const double *z, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = z[i] > 0.0 ? z[i] : 0.0;
}

/* ReLU followed by bfloat16 rounding, the activation handed from one MLP
 * layer to the next (the page's BenchmarkMLP is Linear + ReLU, repeated);
 * the same ReLU as oracle_relu. */
void oracle_relu_bf16(const double *z, int64_t count, uint16_t *h)
{
    for (int64_t i = 0; i < count; ++i) {
        double v = z[i] > 0.0 ? z[i] : 0.0;
        h[i] = oracle_bf16_bits(oracle_bf16_round(v));
    }
}

/* ------------------------------------------------------------------------ */
/* Integer encoding of x for the int8 matrix-core path.  The block planner's */
/* page fixes no encoding of activations for integer arithmetic; the only    */
/* integer cast of activations the pages show (HyperQuant page,              */
/* convert_linears, the int8 LatticeLinear path, another method) is a       */
/* per-token row-absmax int8 cast.  Reading used here, that cast widened to  */
/* two int8 planes:                                                          */
/*   per token (row) m, amax = max_k |x[m,k]| = f * 2^E with f in [0.5, 1);  */
/*   v = round_half_even(x * 2^(14-E)), so |v| <= 2^14 (exact: a power-of-   */
/*       two scaling of a bfloat16 value, rounded once);                     */
/*   hi = floor((v + 128) / 256) in [-64, 64], lo = v - 256*hi in [-128,127];*/
/*   x_hat = v * 2^(E-14), within 2^(E-15) <= amax * 2^-14 of x.             */
/* An all-zero row has v = 0 and exponent 0.  A row holding an Inf or NaN    */
/* gets the exponent OR_XEXP_NONFINITE and zero planes (its outputs are NaN).*/
/* hi, lo: int8 [M][K]; sexp: int32 [M], the exponent E - 14 of x_hat.       */
/* ------------------------------------------------------------------------ */
#define OR_XEXP_NONFINITE (-1000)

void oracle_x_planes(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                     int8_t *hi, int8_t *lo, int32_t *sexp)
{
    for (int64_t m = 0; m < M; ++m) {
        double amax = 0.0;
        int finite = 1;
        for (int64_t k = 0; k < K; ++k) {
            double v = bf16_widen(x[m * ldx + k]);
            if (!isfinite(v)) finite = 0;
            else if (fabs(v) > amax) amax = fabs(v);
        }
        if (!finite) {
            sexp[m] = OR_XEXP_NONFINITE;
            for (int64_t k = 0; k < K; ++k) hi[m * K + k] = lo[m * K + k] = 0;
            continue;
        }
        int E = 0;
        if (amax > 0.0) frexp(amax, &E);
        sexp[m] = amax > 0.0 ? E - 14 : 0;
        for (int64_t k = 0; k < K; ++k) {
            double v = rint(ldexp(bf16_widen(x[m * ldx + k]), 14 - E));
            int32_t iv = (int32_t)v;
            int32_t h = (int32_t)floor((iv + 128) / 256.0);
            hi[m * K + k] = (int8_t)h;
            lo[m * K + k] = (int8_t)(iv - 256 * h);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* W8A8 encoding of x (the opt-in mode with int8 activations).  Per token m   */
/* and 64-wide K-block kb, one int8 code per entry and one power-of-two      */
/* scale:                                                                    */
/*   amax = max over the block of |x| = f * 2^E with f in [0.5, 1);          */
/*   q = clamp(round_half_even(x * 2^(7-E)), -127, 127)  (|x * 2^(7-E)|      */
/*       < 128; the clamp only takes the rounding of values in [127.5, 128)); */
/*   x_hat = q * 2^(E-7), within 2^(E-8) <= amax * 2^-7 of x.                */
/* An all-zero block has codes 0 and exponent 0 (x_hat = 0).  A block        */
/* holding an Inf or NaN gets the exponent OR_XEXP_NONFINITE and zero codes  */
/* (its contributions are NaN).  q: int8 [M][K]; bexp: int32 [M][K/64], the   */
/* exponent E - 7 of the block's scale.                                      */
/* ------------------------------------------------------------------------ */
void oracle_x_w8a8(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                   int8_t *q, int32_t *bexp)
{
    int64_t KB = K / 64;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            const uint16_t *xb = x + m * ldx + 64 * kb;
            int8_t *qb = q + m * K + 64 * kb;
            double amax = 0.0;
            int finite = 1;
            for (int i = 0; i < 64; ++i) {
                double v = bf16_widen(xb[i]);
                if (!isfinite(v)) finite = 0;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            if (!finite) {
                bexp[m * KB + kb] = OR_XEXP_NONFINITE;
                for (int i = 0; i < 64; ++i) qb[i] = 0;
                continue;
            }
            int E = 0;
            if (amax > 0.0) frexp(amax, &E);
            bexp[m * KB + kb] = amax > 0.0 ? E - 7 : 0;
            for (int i = 0; i < 64; ++i) {
                double v = rint(ldexp(bf16_widen(xb[i]), 7 - E));
                if (v > 127.0) v = 127.0;
                if (v < -127.0) v = -127.0;
                qb[i] = (int8_t)v;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Execution buffers: the packed layout (version 1), written out directly    */
/* from its specification.                                                   */
/*                                                                           */
/*  R = row tile (rows per tile), T = ceil(N / R), KB = K / 64.              */
/*  Blocks are enumerated tile by tile, K-block by K-block, row by row:      */
/*  (t, kb, r).  Each format f keeps its own blocks in that order.           */
/*  Regions, each starting at a multiple of 256 bytes, in this order:        */
/*    kbidx  uint32 [5][T*KB + 1]  kbidx[f][t*KB+kb] = number of format-f     */
/*           blocks before (t, kb) in (t, kb) order; the last entry is the    */
/*           total count of format f.                                        */
/*    ids_f  uint16 [c_f] for f = 0..4: kb * R + r                            */
/*    scale_f float [c_f] for f = INT4, INT8: the fp32 scale                  */
/*    pay_f  [c_f][bytes_f] for f = 0..4:                                     */
/*       INT4 32 B: byte j holds element e = 32*(j/16) + (j%16) in its low    */
/*            nibble and element e + 16 in its high nibble, each as the      */
/*            4-bit two's complement of q;                                   */
/*       INT8 64 B: byte i = q_i as an 8-bit two's complement;                */
/*       BF16 / FP16 128 B: the 16-bit patterns, little endian, in order;     */
/*       FP32 256 B: the original fp32 bit patterns.                          */
/* ------------------------------------------------------------------------ */
static const int64_t PAY_BYTES[5] = {32, 64, 128, 128, 256};

static int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

/* offs[0] = kbidx, offs[1..5] = ids_f, offs[6..7] = scale INT4/INT8,
 * offs[8..12] = pay_f; returns the total size in bytes. */
int64_t oracle_pack_layout(int64_t N, int64_t K, int64_t R, const int64_t *counts,
                           int64_t *offs)
{
    int64_t KB = K / OR_BLOCK;
    int64_t T = (N + R - 1) / R;
    int64_t o = 0;
    offs[0] = o; o += align256(5 * (T * KB + 1) * 4);
    for (int f = 0; f < 5; ++f) { offs[1 + f] = o; o += align256(2 * counts[f]); }
    for (int f = 0; f < 2; ++f) { offs[6 + f] = o; o += align256(4 * counts[f]); }
    for (int f = 0; f < 5; ++f) { offs[8 + f] = o; o += align256(PAY_BYTES[f] * counts[f]); }
    return o;
}

/* Fill buf (size from oracle_pack_layout, zero-initialised by the caller). */
void oracle_pack(const float *W, int64_t N, int64_t K, int64_t ldw, const uint8_t *fmt,
                 int64_t R, uint8_t *buf)
{
    int64_t KB = K / OR_BLOCK;
    int64_t T = (N + R - 1) / R;
    int64_t counts[5] = {0, 0, 0, 0, 0};
    for (int64_t i = 0; i < N * KB; ++i) counts[fmt[i]]++;
    int64_t offs[13];
    oracle_pack_layout(N, K, R, counts, offs);
    uint32_t *kbidx = (uint32_t *)(buf + offs[0]);
    int64_t pos[5] = {0, 0, 0, 0, 0};
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            for (int f = 0; f < 5; ++f) kbidx[f * (T * KB + 1) + t * KB + kb] = (uint32_t)pos[f];
            for (int64_t r = 0; r < R; ++r) {
                int64_t n = t * R + r;
                if (n >= N) break;
                const float *w = W + n * ldw + kb * OR_BLOCK;
                int f = fmt[n * KB + kb];
                int64_t p = pos[f]++;
                uint16_t id = (uint16_t)(kb * R + r);
                memcpy(buf + offs[1 + f] + 2 * p, &id, 2);
                uint8_t *dst = buf + offs[8 + f] + PAY_BYTES[f] * p;
                if (f == OR_INT4 || f == OR_INT8) {
                    float s;
                    int8_t q[OR_BLOCK];
                    oracle_int_quant_block(w, f == OR_INT4 ? 7 : 127, &s, q);
                    memcpy(buf + offs[6 + f] + 4 * p, &s, 4);
                    if (f == OR_INT8) {
                        for (int i = 0; i < OR_BLOCK; ++i) dst[i] = (uint8_t)q[i];
                    } else {
                        for (int j = 0; j < 32; ++j) {
                            int e = 32 * (j / 16) + (j % 16);
                            dst[j] = (uint8_t)((q[e] & 15) | ((q[e + 16] & 15) << 4));
                        }
                    }
                } else if (f == OR_BF16) {
                    for (int i = 0; i < OR_BLOCK; ++i) {
                        uint16_t b = oracle_bf16_bits(oracle_bf16_round((double)w[i]));
                        memcpy(dst + 2 * i, &b, 2);
                    }
                } else if (f == OR_FP16) {
                    for (int i = 0; i < OR_BLOCK; ++i) {
                        uint16_t b = oracle_fp16_bits(oracle_fp16_round((double)w[i]));
                        memcpy(dst + 2 * i, &b, 2);
                    }
                } else {
                    memcpy(dst, w, 256);
                }
            }
        }
    }
    for (int f = 0; f < 5; ++f) kbidx[f * (T * KB + 1) + T * KB] = (uint32_t)pos[f];
}
