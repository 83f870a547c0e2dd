"""GPU parity of the MFMA path (HT_PATH_GEMM) against the CPU oracle.

Bar: max|y_gpu - y_oracle| <= 1e-3 * max|y_oracle| with identical bfloat16
activations (oracle in fp64).  Shapes span several 128 x 64 output tiles with
ragged edges in M and N, every format, every row tile, ReLU and row strides.
"""
import numpy as np
import pytest
import torch

from block_planner_amd import api
from block_planner_amd import binding as B
from block_planner_amd import workloads as wl

pytestmark = pytest.mark.gpu

INT4, INT8, BF16, FP16, FP32 = 0, 1, 2, 3, 4
TOL = 1e-3
GEMM = B.HT_PATH_GEMM


def dev():
    return torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_gpu(xbits):
    return gpu(xbits.view(np.int16)).view(torch.bfloat16)


def check_close(y_gpu, y_or, what=""):
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.max(np.abs(y_gpu - y_or))
    ref = np.max(np.abs(y_or))
    assert np.all(np.isfinite(y_gpu)), what
    assert err <= TOL * ref, f"{what}: max|dy| = {err:.3e} > {TOL} * {ref:.3e}"
    return err / max(ref, 1e-300)


def run_gemm(W, fmt, xbits, R=16, act=0, ldx_pad=0, ldy_pad=0, path=GEMM):
    pw = api.pack(gpu(W), gpu(fmt), row_tile=R)
    M, K = xbits.shape
    xs = torch.zeros((M, K + ldx_pad), dtype=torch.bfloat16, device=dev())
    xs[:, :K] = bf16_gpu(xbits)
    ys = torch.full((M, W.shape[0] + ldy_pad), 7.0, dtype=torch.float32, device=dev())
    x_v, y_v = xs[:, :K], ys[:, :W.shape[0]]
    api.linear(pw, x_v, act=act, out=y_v, path=path)
    torch.cuda.synchronize()
    if ldy_pad:
        assert torch.all(ys[:, W.shape[0]:] == 7.0)   # padding untouched
    return y_v.cpu().numpy()


@pytest.mark.parametrize("M", [1, 7, 33, 64, 130, 257])
def test_gemm_small_weight(orc, M):
    W = wl.small_weight()
    fmt = orc.plan(W)
    x = wl.to_bf16_bits(wl.small_activation(m=M))
    check_close(run_gemm(W, fmt, x), orc.linear(W, fmt, x), f"M={M}")


@pytest.mark.parametrize("R", [1, 2, 4, 8, 16])
def test_gemm_all_formats(orc, R):
    rng = np.random.default_rng(27)
    W = (rng.normal(size=(200, 512)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(200, 8)).astype(np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(150, 512)).astype(np.float32))
    check_close(run_gemm(W, fmt, x, R=R), orc.linear(W, fmt, x), f"R={R}")


@pytest.mark.parametrize("force", [INT4, INT8, BF16, FP16, FP32])
def test_gemm_single_format(orc, force):
    W = wl.small_weight(seed=4)
    fmt = orc.plan(W, force=force)
    x = wl.to_bf16_bits(wl.small_activation(m=96))
    check_close(run_gemm(W, fmt, x), orc.linear(W, fmt, x), f"force={force}")


def test_gemm_fp32_entries_keep_16_bits(orc):
    """FP32 blocks whose values are not bfloat16-exact: one bf16 plane alone
    would miss the tolerance; hi + lo keeps 16 significant bits."""
    rng = np.random.default_rng(28)
    W = (1.0 + rng.uniform(-2 ** -8, 2 ** -8, size=(64, 256))).astype(np.float32)
    W[:, ::2] *= -1.0
    fmt = np.full((64, 4), FP32, np.uint8)
    x = wl.to_bf16_bits(np.ones((64, 256), np.float32))
    y = run_gemm(W, fmt, x)
    y_or = orc.linear(W, fmt, x)
    # the sums cancel to ~1e-1 while the entries are ~1: a tight check
    assert np.max(np.abs(y - y_or)) <= 1e-5 * np.max(np.abs(W)) * 256


def test_gemm_relu_strides_ragged(orc):
    rng = np.random.default_rng(29)
    W = (rng.normal(size=(37, 192)) * 0.1).astype(np.float32)
    fmt = orc.plan(W, eps_int4=0.2)
    x = wl.to_bf16_bits(rng.normal(size=(70, 192)).astype(np.float32))
    y = run_gemm(W, fmt, x, act=1, ldx_pad=64, ldy_pad=5)
    check_close(y, np.maximum(orc.linear(W, fmt, x), 0), "relu/strides")


def test_gemm_matches_gemv_path(orc):
    """The two paths over the same packed weight agree within the bar."""
    W = wl.mlp_weight(2, dim=4096)[:512]
    fmt = orc.plan(W)
    x = wl.to_bf16_bits(wl.mlp_activation(8)[:, :4096])
    y_gemm = run_gemm(W, fmt, x)
    y_gemv = run_gemm(W, fmt, x, path=B.HT_PATH_GEMV)
    check_close(y_gemm, orc.linear(W, fmt, x), "gemm")
    check_close(y_gemv, orc.linear(W, fmt, x), "gemv")


def test_gemm_deterministic():
    W = wl.mlp_weight(1, dim=4096)[:1024]
    Wg = gpu(W)
    fmt = api.plan(Wg)
    pw = api.pack(Wg, fmt)
    x = bf16_gpu(wl.to_bf16_bits(wl.activation("llama8b", 200, 4096)))
    y1 = api.linear(pw, x, path=GEMM).clone()
    y2 = api.linear(pw, x, path=GEMM).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("name", ["q", "k", "gate", "down"])
def test_gemm_prefill_full_size_sampled(orc, name):
    """Llama-8B-shaped layers at the prefill batch (M = 2048): sampled outputs
    against the oracle, one by one."""
    shp = [s for s in wl.llama8b_shapes() if s.name == name][0]
    W = wl.llama8b_weight(0, shp)
    fmt_or = orc.plan(W)
    Wg = gpu(W)
    fmt = api.plan(Wg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fmt.cpu().numpy(), fmt_or)
    pw = api.pack(Wg, fmt)
    del Wg
    M = 2048
    x = wl.to_bf16_bits(wl.activation("llama8b", M, shp.k))
    y = api.linear(pw, bf16_gpu(x))      # AUTO takes the MFMA path at this M
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    mi = rng.integers(0, M, size=192)
    ni = rng.integers(0, shp.n, size=192)
    mi[:2] = [0, M - 1]
    ni[:2] = [0, shp.n - 1]
    ys = orc.linear_sampled(W, fmt_or, x, mi, ni)
    assert np.max(np.abs(y.cpu().numpy()[mi, ni] - ys)) <= TOL * np.max(np.abs(ys)), name


@pytest.mark.parametrize("M,N,K", [(16, 512, 14336), (32, 200, 1024), (33, 96, 64 * 37)])
def test_gemm_split_k(orc, M, N, K):
    """Few output tiles: K is split across workgroups (ragged last split) and a
    second kernel adds the splits in order; bitwise reproducible."""
    shp = wl.LinearShape("t", N, K)
    W = wl.llama8b_weight(1, shp)
    fmt = orc.plan(W)
    pw = api.pack(gpu(W), gpu(fmt))
    assert B.ht_linear_workspace(pw.desc, M, GEMM) > 0
    x = wl.to_bf16_bits(wl.activation("llama8b", M, K, seed=2))
    y = run_gemm(W, fmt, x)
    check_close(y, orc.linear(W, fmt, x), f"M={M} N={N} K={K}")
    xg = bf16_gpu(x)
    y1 = api.linear(pw, xg, path=GEMM).clone()
    y2 = api.linear(pw, xg, path=GEMM).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
