"""CPU oracle of the per-block mixed-precision linear -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The library itself never calls it and shares no
code with it.  The arithmetic lives in ``ht_oracle.c`` (plain C, compiled with
``-O2 -ffp-contract=off``, no fast-math); this module only marshals numpy
arrays into it.

Format codes: 0 INT4, 1 INT8, 2 BF16, 3 FP16, 4 FP32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

INT4, INT8, BF16, FP16, FP32 = 0, 1, 2, 3, 4
FORMATS = ("INT4", "INT8", "BF16", "FP16", "FP32")
BLOCK_K = 64
PAY_BYTES = (32, 64, 128, 128, 256)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ht_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile the oracle into oracle/liboracle.so (always recompiles)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", _SRC, "-o", _LIB, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    D = ctypes.c_double
    I = ctypes.c_int
    lib.oracle_bf16_round.restype = D
    lib.oracle_bf16_round.argtypes = [D]
    lib.oracle_fp16_round.restype = D
    lib.oracle_fp16_round.argtypes = [D]
    lib.oracle_bf16_bits.restype = ctypes.c_uint16
    lib.oracle_bf16_bits.argtypes = [D]
    lib.oracle_fp16_bits.restype = ctypes.c_uint16
    lib.oracle_fp16_bits.argtypes = [D]
    lib.oracle_block_err2.restype = D
    lib.oracle_block_err2.argtypes = [P, I]
    lib.oracle_block_nrm2.restype = D
    lib.oracle_block_nrm2.argtypes = [P]
    lib.oracle_pick_block.restype = I
    lib.oracle_pick_block.argtypes = [P, P, I, I]
    lib.oracle_int_quant_block.restype = None
    lib.oracle_int_quant_block.argtypes = [P, I, P, P]
    lib.oracle_plan.restype = None
    lib.oracle_plan.argtypes = [P, I64, I64, I64, D, D, D, D, I, I, P]
    lib.oracle_block_errors.restype = None
    lib.oracle_block_errors.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_int_quant.restype = None
    lib.oracle_int_quant.argtypes = [P, I64, I64, I64, I, P, P]
    lib.oracle_dequant.restype = None
    lib.oracle_dequant.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_linear.restype = None
    lib.oracle_linear.argtypes = [P, I64, I64, I64, P, P, I64, I64, P, I64]
    lib.oracle_linear_sampled.restype = None
    lib.oracle_linear_sampled.argtypes = [P, I64, I64, P, P, I64, P, P, I64, P]
    lib.oracle_relu.restype = None
    lib.oracle_relu.argtypes = [P, I64, P]
    lib.oracle_relu_bf16.restype = None
    lib.oracle_relu_bf16.argtypes = [P, I64, P]
    lib.oracle_x_planes.restype = None
    lib.oracle_x_planes.argtypes = [P, I64, I64, I64, P, P, P]
    lib.oracle_x_w8a8.restype = None
    lib.oracle_x_w8a8.argtypes = [P, I64, I64, I64, P, P]
    lib.oracle_pack_layout.restype = I64
    lib.oracle_pack_layout.argtypes = [I64, I64, I64, P, P]
    lib.oracle_pack.restype = None
    lib.oracle_pack.argtypes = [P, I64, I64, I64, P, I64, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _w(W: np.ndarray) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.float32)
    assert W.ndim == 2 and W.shape[1] % BLOCK_K == 0, W.shape
    return W


DEFAULT_EPS = dict(eps_int4=0.08, eps_int8=0.01, eps_bf16=0.0, eps_fp16=0.0)


# --- scalar helpers ---------------------------------------------------------
def bf16_round(v: float) -> float:
    return _load().oracle_bf16_round(float(v))


def fp16_round(v: float) -> float:
    return _load().oracle_fp16_round(float(v))


def bf16_bits(v: float) -> int:
    return int(_load().oracle_bf16_bits(float(v)))


def fp16_bits(v: float) -> int:
    return int(_load().oracle_fp16_bits(float(v)))


# --- block level ------------------------------------------------------------
def block_err2(w: np.ndarray, fmt: int) -> float:
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.shape == (BLOCK_K,)
    return _load().oracle_block_err2(_ptr(w), int(fmt))


def block_nrm2(w: np.ndarray) -> float:
    w = np.ascontiguousarray(w, dtype=np.float32)
    return _load().oracle_block_nrm2(_ptr(w))


def int_quant_block(w: np.ndarray, Q: int):
    w = np.ascontiguousarray(w, dtype=np.float32)
    s = np.zeros(1, np.float32)
    q = np.zeros(BLOCK_K, np.int8)
    _load().oracle_int_quant_block(_ptr(w), int(Q), _ptr(s), _ptr(q))
    return s[0], q


def pick_block(w: np.ndarray, eps_int4=0.08, eps_int8=0.01, eps_bf16=0.0, eps_fp16=0.0,
               prefer_bf16=True, force=-1) -> int:
    w = np.ascontiguousarray(w, dtype=np.float32)
    eps = np.array([eps_int4, eps_int8, eps_bf16, eps_fp16], np.float64)
    return _load().oracle_pick_block(_ptr(w), _ptr(eps), int(bool(prefer_bf16)), int(force))


# --- matrix level -----------------------------------------------------------
def plan(W: np.ndarray, eps_int4=0.08, eps_int8=0.01, eps_bf16=0.0, eps_fp16=0.0,
         prefer_bf16=True, force=-1) -> np.ndarray:
    """Format map uint8 [N, K/64]."""
    W = _w(W)
    N, K = W.shape
    fmt = np.zeros((N, K // BLOCK_K), np.uint8)
    _load().oracle_plan(_ptr(W), N, K, K, float(eps_int4), float(eps_int8), float(eps_bf16),
                        float(eps_fp16), int(bool(prefer_bf16)), int(force), _ptr(fmt))
    return fmt


def block_errors(W: np.ndarray):
    """(err2 [N, K/64, 5], nrm2 [N, K/64]) in double."""
    W = _w(W)
    N, K = W.shape
    err2 = np.zeros((N, K // BLOCK_K, 5), np.float64)
    nrm2 = np.zeros((N, K // BLOCK_K), np.float64)
    _load().oracle_block_errors(_ptr(W), N, K, K, _ptr(err2), _ptr(nrm2))
    return err2, nrm2


def int_quant(W: np.ndarray, Q: int):
    """(scale float32 [N, K/64], codes int8 [N, K]) for every block."""
    W = _w(W)
    N, K = W.shape
    scale = np.zeros((N, K // BLOCK_K), np.float32)
    codes = np.zeros((N, K), np.int8)
    _load().oracle_int_quant(_ptr(W), N, K, K, int(Q), _ptr(scale), _ptr(codes))
    return scale, codes


def dequant(W: np.ndarray, fmt: np.ndarray) -> np.ndarray:
    W = _w(W)
    N, K = W.shape
    fmt = np.ascontiguousarray(fmt, dtype=np.uint8)
    assert fmt.shape == (N, K // BLOCK_K)
    out = np.zeros((N, K), np.float64)
    _load().oracle_dequant(_ptr(W), N, K, K, _ptr(fmt), _ptr(out))
    return out


def linear(W: np.ndarray, fmt: np.ndarray, x_bf16: np.ndarray) -> np.ndarray:
    """y [M, N] (double) = x_hat [M, K] . W_hat^T; x given as bfloat16 bits."""
    W = _w(W)
    N, K = W.shape
    fmt = np.ascontiguousarray(fmt, dtype=np.uint8)
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    assert x.ndim == 2 and x.shape[1] == K
    M = x.shape[0]
    y = np.zeros((M, N), np.float64)
    _load().oracle_linear(_ptr(W), N, K, K, _ptr(fmt), _ptr(x), M, K, _ptr(y), N)
    return y


def linear_sampled(W: np.ndarray, fmt: np.ndarray, x_bf16: np.ndarray, m_idx, n_idx) -> np.ndarray:
    W = _w(W)
    N, K = W.shape
    fmt = np.ascontiguousarray(fmt, dtype=np.uint8)
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    y = np.zeros(mi.size, np.float64)
    _load().oracle_linear_sampled(_ptr(W), K, K, _ptr(fmt), _ptr(x), K, _ptr(mi), _ptr(ni),
                                  mi.size, _ptr(y))
    return y


def linear_backward_data(W: np.ndarray, fmt: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """dX [M, K] (double) = dY . W_hat: the input gradient of y = x . W_hat^T
    (the pages' training support), dY given in fp32 and widened exactly."""
    dy = np.ascontiguousarray(dy, dtype=np.float32).astype(np.float64)
    assert dy.ndim == 2 and dy.shape[1] == W.shape[0]
    return dy @ dequant(W, fmt)


def linear_backward_weight(dy: np.ndarray, x_bf16: np.ndarray) -> np.ndarray:
    """dW [N, K] (double) = dY^T . x: the gradient for the fp32 master weight
    under the straight-through estimator (the gradient of W_hat passed to W
    unchanged), x being the bf16 activations the forward consumed and dY the
    fp32 output gradient, both widened exactly (the pages' training support
    with an STE)."""
    dy = np.ascontiguousarray(dy, dtype=np.float32).astype(np.float64)
    xb = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    assert dy.ndim == 2 and xb.ndim == 2 and dy.shape[0] == xb.shape[0]
    x = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return dy.T @ x


def relu(z: np.ndarray) -> np.ndarray:
    """max(z, 0) in double with zero, negative values and NaN all giving +0."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    out = np.zeros(z.shape, np.float64)
    _load().oracle_relu(_ptr(z), z.size, _ptr(out))
    return out


def relu_bf16(z: np.ndarray) -> np.ndarray:
    """bfloat16 bits of max(z, 0), round to nearest even."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    h = np.zeros(z.shape, np.uint16)
    _load().oracle_relu_bf16(_ptr(z), z.size, _ptr(h))
    return h


def mlp(weights, fmts, x_bf16: np.ndarray):
    """Linear + ReLU per layer; bfloat16 activations between layers, the last
    layer's ReLU output in double.  Returns (y, [h_1 .. h_{L-1}] as bf16 bits)."""
    h = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    hs = []
    for li, (W, f) in enumerate(zip(weights, fmts)):
        z = linear(W, f, h)
        if li + 1 < len(weights):
            h = relu_bf16(z)
            hs.append(h)
        else:
            return relu(z), hs
    raise ValueError("no layers")


# --- integer encoding of x (int8 matrix-core path) -------------------------
XEXP_NONFINITE = -1000


def x_planes(x_bf16: np.ndarray):
    """(hi, lo, sexp): x[m, k] ~ (256 * hi + lo) * 2^sexp[m], two int8 planes
    per token (the encoding's definition is in ht_oracle.c)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    assert x.ndim == 2
    M, K = x.shape
    hi = np.zeros((M, K), np.int8)
    lo = np.zeros((M, K), np.int8)
    sexp = np.zeros(M, np.int32)
    _load().oracle_x_planes(_ptr(x), M, K, K, _ptr(hi), _ptr(lo), _ptr(sexp))
    return hi, lo, sexp


def x_hat(hi: np.ndarray, lo: np.ndarray, sexp: np.ndarray) -> np.ndarray:
    """The encoded x in double; rows marked non-finite are NaN."""
    v = 256.0 * hi.astype(np.float64) + lo.astype(np.float64)
    ok = sexp != XEXP_NONFINITE
    out = np.ldexp(v, np.where(ok, sexp, 0)[:, None])
    out[~ok] = np.nan
    return out


def linear_xplanes(W: np.ndarray, fmt: np.ndarray, x_bf16: np.ndarray) -> np.ndarray:
    """y [M, N] (double) = x_hat . W_hat^T with x_hat the two-plane encoding of
    x: what the int8 matrix-core path computes, before fp32 rounding."""
    return x_hat(*x_planes(x_bf16)) @ dequant(W, fmt).T


def x_w8a8(x_bf16: np.ndarray):
    """(q, bexp): x[m, k] ~ q[m, k] * 2^bexp[m, k // 64], one int8 code per
    entry and one power-of-two scale per token and 64-wide K-block (the W8A8
    encoding; its definition is in ht_oracle.c)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    assert x.ndim == 2 and x.shape[1] % BLOCK_K == 0
    M, K = x.shape
    q = np.zeros((M, K), np.int8)
    bexp = np.zeros((M, K // BLOCK_K), np.int32)
    _load().oracle_x_w8a8(_ptr(x), M, K, K, _ptr(q), _ptr(bexp))
    return q, bexp


def x_hat_w8a8(q: np.ndarray, bexp: np.ndarray) -> np.ndarray:
    """The W8A8-encoded x in double; blocks marked non-finite are NaN."""
    ok = bexp != XEXP_NONFINITE
    e = np.repeat(np.where(ok, bexp, 0), BLOCK_K, axis=1)
    out = np.ldexp(q.astype(np.float64), e)
    out[~np.repeat(ok, BLOCK_K, axis=1)] = np.nan
    return out


def linear_w8a8(W: np.ndarray, fmt: np.ndarray, x_bf16: np.ndarray) -> np.ndarray:
    """y [M, N] (double) = x_hat . W_hat^T with x_hat the W8A8 encoding of x:
    what the W8A8 mode computes on its integer tiles, before fp32 rounding."""
    return x_hat_w8a8(*x_w8a8(x_bf16)) @ dequant(W, fmt).T


def pack_layout(N: int, K: int, R: int, counts) -> tuple[int, list[int]]:
    c = np.ascontiguousarray(counts, dtype=np.int64)
    offs = np.zeros(13, np.int64)
    size = _load().oracle_pack_layout(N, K, R, _ptr(c), _ptr(offs))
    return int(size), [int(v) for v in offs]


def pack(W: np.ndarray, fmt: np.ndarray, R: int) -> np.ndarray:
    """The packed execution buffer (uint8) of layout version 1."""
    W = _w(W)
    N, K = W.shape
    fmt = np.ascontiguousarray(fmt, dtype=np.uint8)
    counts = np.bincount(fmt.reshape(-1), minlength=5).astype(np.int64)
    size, _ = pack_layout(N, K, R, counts)
    buf = np.zeros(size, np.uint8)
    _load().oracle_pack(_ptr(W), N, K, K, _ptr(fmt), int(R), _ptr(buf))
    return buf
