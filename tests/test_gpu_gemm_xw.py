"""GPU parity of the two-pass prefill GEMM (weight tiles expanded once into
bfloat16 planes, then the matrix-core kernel on them), which HT_PATH_GEMM
takes from 1024 rows when the 256 x 128 output tiles fill the chip.

Bars:
- against the fused prefill kernel (same planes and scales; the lo plane's
  products join the sum once at the end instead of per step): within
  1e-5 * max|y|, row by row (rows of y depend only on their row of x, so
  the fused kernel's run on the first 1000 rows is the reference);
- against the CPU oracle (fp64): max|y - y_oracle| <= 1e-3 * max|y_oracle|
  over every output, ragged N and M, every format, row tiles 16 and 4;
- the bfloat16 ReLU output of the MLP's per-layer path equals
  bf16_rne(relu(y)) of the fp32 output, bit for bit;
- two calls give the same bits.
"""
import numpy as np
import pytest
import torch

from block_planner_amd import api
from block_planner_amd import binding as B
from block_planner_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 1e-3
GEMM = B.HT_PATH_GEMM


def dev():
    return torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_gpu(xbits):
    return gpu(xbits.view(np.int16)).view(torch.bfloat16)


def mixed_weight(rng, N, K):
    """Student-t weights, 0.5% of the columns scaled by 8, and a format map
    drawn per block from all five formats (INT8 most often)."""
    W = (rng.standard_t(4, size=(N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, size=max(1, K // 200), replace=False)] *= np.float32(8.0)
    fmt = rng.choice(5, size=(N, K // 64), p=[0.1, 0.6, 0.1, 0.1, 0.1]).astype(np.uint8)
    return W, fmt


def linear(pw, xbits, act=B.HT_ACT_NONE):
    y = api.linear(pw, bf16_gpu(xbits), act=act, path=GEMM)
    torch.cuda.synchronize()
    return y


def test_xw_agrees_with_fused_kernel_and_repeats():
    """6144 x 1024: at 1000 rows (4 row tiles, 192 output tiles, no K-split)
    the fused kernel runs; at 1024 rows the two-pass path.  The two differ
    only in when the lo plane's products join the sum (per step, or once at
    the end), so their first 1000 rows agree to fp32 rounding: within
    1e-5 * max|y| (100 times tighter than the oracle bar).  A second
    two-pass call repeats its bits."""
    rng = np.random.default_rng(501)
    W, fmt = mixed_weight(rng, 6144, 1024)
    pw = api.pack(gpu(W), gpu(fmt))
    x = wl.to_bf16_bits(rng.normal(size=(1024, 1024)).astype(np.float32))
    assert B.ht_linear_workspace(pw.desc, 1000, GEMM) < B.ht_linear_workspace(pw.desc, 1024, GEMM)
    y_fused = linear(pw, x[:1000])
    y_xw = linear(pw, x)
    d = (y_xw[:1000] - y_fused).abs().max().item()
    assert d <= 1e-5 * y_fused.abs().max().item()
    assert torch.equal(linear(pw, x), y_xw)


@pytest.mark.parametrize("R", [16, 4])
def test_xw_matches_oracle_ragged(orc, R):
    """N = 6000 (a ragged last column tile), K = 640, M = 1100 (a ragged
    last row tile), every format, row tile R; every output against fp64."""
    rng = np.random.default_rng(510 + R)
    W, fmt = mixed_weight(rng, 6000, 640)
    pw = api.pack(gpu(W), gpu(fmt), row_tile=R)
    x = wl.to_bf16_bits(rng.normal(size=(1100, 640)).astype(np.float32))
    y = linear(pw, x).cpu().numpy().astype(np.float64)
    ref = orc.linear(W, fmt, x)
    assert np.all(np.isfinite(y))
    err = np.max(np.abs(y - ref))
    assert err <= TOL * np.max(np.abs(ref)), f"R={R}: {err:.3e} vs {np.max(np.abs(ref)):.3e}"


def test_xw_relu_bf16_output_and_strides(orc):
    """Row strides (ldx = K + 8, ldy = N + 4, padding untouched), ReLU, and
    the MLP's per-layer path: its bfloat16 hidden activation is exactly
    bf16_rne(relu(y)) of the fp32 two-pass output."""
    rng = np.random.default_rng(520)
    N, K, M = 6144, 512, 1024
    W, fmt = mixed_weight(rng, N, K)
    W2 = (rng.standard_t(4, size=(256, N)) * 0.02).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    pw2 = api.pack(gpu(W2), gpu(orc.plan(W2)))
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    xs = torch.zeros((M, K + 8), dtype=torch.bfloat16, device=dev())
    xs[:, :K] = bf16_gpu(x)
    ys = torch.full((M, N + 4), 7.0, dtype=torch.float32, device=dev())
    api.linear(pw, xs[:, :K], act=B.HT_ACT_RELU, out=ys[:, :N], path=GEMM)
    torch.cuda.synchronize()
    assert torch.all(ys[:, N:] == 7.0)
    ref = np.maximum(orc.linear(W, fmt, x), 0.0)
    y = ys[:, :N].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(y - ref)) <= TOL * np.max(np.abs(ref))
    # the per-layer MLP writes the hidden layer as bfloat16 from the same kernel
    ws = api.mlp_workspace([pw, pw2], M, dev())
    _, dumps = api.mlp([pw, pw2], bf16_gpu(x), dump=True, ws=ws, path=B.HT_PATH_AUTO)
    torch.cuda.synchronize()
    h_ref = ys[:, :N].contiguous().to(torch.bfloat16)          # round to nearest even
    assert torch.equal(dumps[0].view(torch.int16), h_ref.view(torch.int16))


def test_xw_smaller_workspace_runs_single_pass():
    """Given less workspace than the records need (here none: 6144 x 1024
    at 1024 rows has no K-split partials) HT_PATH_GEMM runs the single-pass
    kernel: bitwise that kernel's result at 1000 rows on the shared rows, and
    within 1e-5 * max|y| of the two-pass result."""
    rng = np.random.default_rng(502)
    W, fmt = mixed_weight(rng, 6144, 1024)
    pw = api.pack(gpu(W), gpu(fmt))
    x = wl.to_bf16_bits(rng.normal(size=(1024, 1024)).astype(np.float32))
    assert B.ht_linear_workspace(pw.desc, 1000, GEMM) == 0
    y_small = torch.empty((1024, 6144), dtype=torch.float32, device=dev())
    B.ht_linear_forward(pw.desc, bf16_gpu(x), y_small, path=GEMM, ws=None)
    y_1000 = linear(pw, x[:1000])
    y_xw = linear(pw, x)
    assert torch.equal(y_small[:1000], y_1000)
    assert (y_small - y_xw).abs().max().item() <= 1e-5 * y_xw.abs().max().item()


@pytest.mark.parametrize("act", [B.HT_ACT_NONE, B.HT_ACT_RELU])
def test_xw_split_last_round(orc, act):
    """36 x 8 = 288 output tiles: the last round's 32 tiles run as two
    workgroups each over the K halves and a second kernel adds the halves
    (first, then second) and applies the activation.  N = 4600 (ragged last
    column tile), M = 2040 (ragged last row tile), K = 256: every output
    against fp64, and the first 1000 rows against the single-pass kernel
    within 1e-5 * max|y|."""
    rng = np.random.default_rng(530 + act)
    W, fmt = mixed_weight(rng, 4600, 256)
    pw = api.pack(gpu(W), gpu(fmt))
    x = wl.to_bf16_bits(rng.normal(size=(2040, 256)).astype(np.float32))
    y = api.linear(pw, bf16_gpu(x), act=act, path=GEMM)
    torch.cuda.synchronize()
    ref = orc.linear(W, fmt, x)
    if act == B.HT_ACT_RELU:
        ref = np.maximum(ref, 0.0)
    yc = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yc))
    assert np.max(np.abs(yc - ref)) <= TOL * np.max(np.abs(ref))
    y1 = api.linear(pw, bf16_gpu(x[:1000]), act=act, path=GEMM)
    torch.cuda.synchronize()
    assert (y[:1000] - y1).abs().max().item() <= 1e-5 * y1.abs().max().item()
    assert torch.equal(api.linear(pw, bf16_gpu(x), act=act, path=GEMM), y)
