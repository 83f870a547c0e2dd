"""GPU parity of the register-dequantising MFMA path (HT_PATH_GEMV_MFMA)
against the CPU oracle.

Bar: max|y_gpu - y_oracle| <= 1e-3 * max|y_oracle| with identical bfloat16
activations (oracle in fp64).  Cases: the small configuration at batch 1 to
70 (one, two and three 32-row launches), every format mixed and forced, a row
count that is not a multiple of 16, K-splits (few row tiles), a wavefront
with 15 K-blocks, row strides and ReLU, full-size decode layers, and the
row-tile restriction.
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
DEC = B.HT_PATH_GEMV_MFMA


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


def run_dec(W, fmt, xbits, act=0, ldx_pad=0, ldy_pad=0):
    print(f"gemv_mfma case: W {W.shape} M {xbits.shape[0]} act {act} pads {ldx_pad},{ldy_pad}", flush=True)
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    M, K = xbits.shape
    xs = torch.zeros((M, K + ldx_pad), dtype=torch.bfloat16, device=dev())
    xs[:, :K] = bf16_gpu(xbits)
    ys = torch.full((M, W.shape[0] + ldy_pad), 7.0, dtype=torch.float32, device=dev())
    x_v, y_v = xs[:, :K], ys[:, :W.shape[0]]
    api.linear(pw, x_v, act=act, out=y_v, path=DEC)
    torch.cuda.synchronize()
    if ldy_pad:
        assert torch.all(ys[:, W.shape[0]:] == 7.0)   # padding untouched
    return y_v.cpu().numpy()


def relu(y):
    return np.maximum(y, 0.0)


@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 33, 64, 70])
def test_dec_small_weight(orc, M):
    W = wl.small_weight()
    fmt = orc.plan(W)
    x = wl.to_bf16_bits(wl.small_activation(m=M))
    check_close(run_dec(W, fmt, x), orc.linear(W, fmt, x), f"M={M}")


def test_dec_all_formats_ragged_rows(orc):
    rng = np.random.default_rng(31)
    W = (rng.normal(size=(200, 512)) * 0.05).astype(np.float32)    # 12.5 row tiles
    fmt = rng.integers(0, 5, size=(200, 8)).astype(np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(37, 512)).astype(np.float32))
    check_close(run_dec(W, fmt, x), orc.linear(W, fmt, x), "mixed")


@pytest.mark.parametrize("force", [INT4, INT8, BF16, FP16, FP32])
def test_dec_single_format(orc, force):
    W = wl.small_weight(seed=4)
    fmt = orc.plan(W, force=force)
    x = wl.to_bf16_bits(wl.small_activation(m=24))
    check_close(run_dec(W, fmt, x), orc.linear(W, fmt, x), f"force={force}")


@pytest.mark.parametrize("N,K,M", [(40, 4096, 3), (256, 14336, 16), (48, 1024, 32)])
def test_dec_k_split(orc, N, K, M):
    """Few row tiles: the K range is split over workgroups and a second
    kernel adds the splits (ReLU applied there)."""
    rng = np.random.default_rng(N + K + M)
    W = (rng.standard_t(4, size=(N, K)) / 64).astype(np.float32)
    fmt = rng.integers(0, 5, size=(N, K // 64)).astype(np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    check_close(run_dec(W, fmt, x, act=1), relu(orc.linear(W, fmt, x)), f"N={N} K={K}")


def test_dec_fifteen_blocks_per_wave(orc):
    """192 row tiles and K = 15360: no split, each wavefront walks 15 K-blocks
    (the whole K-block index window)."""
    rng = np.random.default_rng(15)
    N, K = 3072, 15360
    W = (rng.normal(size=(N, K)) * 0.02).astype(np.float32)
    fmt = rng.integers(0, 5, size=(N, K // 64)).astype(np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(2, K)).astype(np.float32))
    check_close(run_dec(W, fmt, x), orc.linear(W, fmt, x), "K=15360")


def test_dec_strides_relu(orc):
    W = wl.small_weight(seed=9)
    fmt = orc.plan(W)
    x = wl.to_bf16_bits(wl.small_activation(m=20))
    y = run_dec(W, fmt, x, act=1, ldx_pad=64, ldy_pad=5)
    check_close(y, relu(orc.linear(W, fmt, x)), "strides")
    assert np.all(y >= 0)


def test_dec_reproducible():
    W = wl.small_weight(seed=2)
    rng = np.random.default_rng(2)
    fmt = rng.integers(0, 5, size=(W.shape[0], W.shape[1] // 64)).astype(np.uint8)
    x = wl.to_bf16_bits(wl.small_activation(m=32))
    a = run_dec(W, fmt, x)
    b = run_dec(W, fmt, x)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("M", [16, 32])
def test_dec_mlp_layer_full(orc, M):
    """A 4096 x 4096 layer of the benchmark MLP (planned by the oracle) at
    batch 16 and 32, every output against the oracle."""
    W = wl.mlp_weight(1)
    fmt = orc.plan(W)
    x = wl.to_bf16_bits(np.random.default_rng(M).normal(size=(M, 4096)).astype(np.float32))
    check_close(run_dec(W, fmt, x), orc.linear(W, fmt, x), f"mlp layer M={M}")


@pytest.mark.parametrize("name", ["gate", "down"])
def test_dec_llama8b_full(orc, name):
    """Llama-8B-shaped gate (14336 x 4096) and down (4096 x 14336, 14
    K-blocks per wavefront) projections at batch 16."""
    shp = [s for s in wl.llama8b_shapes() if s.name == name][0]
    W = wl.llama8b_weight(0, shp)
    fmt = orc.plan(W)
    x = wl.to_bf16_bits(wl.activation("llama8b", 16, shp.k, seed=5))
    check_close(run_dec(W, fmt, x), orc.linear(W, fmt, x), f"llama8b.{name} M=16")


def test_dec_needs_row_tile_16():
    W = wl.small_weight()
    fmt = np.zeros((W.shape[0], W.shape[1] // 64), np.uint8)
    pw = api.pack(gpu(W), gpu(fmt), row_tile=8)
    x = torch.zeros((4, W.shape[1]), dtype=torch.bfloat16, device=dev())
    y = torch.empty((4, W.shape[0]), dtype=torch.float32, device=dev())
    with pytest.raises(B.HTError):
        B.ht_linear_workspace(pw.desc, 4, DEC)
    with pytest.raises(B.HTError):
        B.ht_linear_forward(pw.desc, x, y, path=DEC)


@pytest.mark.parametrize("seed", range(8))
def test_dec_random_shapes(orc, seed):
    """Seeded random shapes: rows from 1 to 600 (ragged last tile), 1 to 300
    K-blocks (a partial last round of 64 or 32 K-blocks, K-splits when there
    are few row tiles), 1 to 40 rows of x, random formats, ReLU half the
    time."""
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.integers(1, 601))
    KB = int(rng.integers(1, 301))
    M = int(rng.integers(1, 41))
    act = int(rng.integers(0, 2))
    W = (rng.standard_t(4, size=(N, 64 * KB)) * 0.03).astype(np.float32)
    fmt = rng.integers(0, 5, size=(N, KB)).astype(np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(M, 64 * KB)).astype(np.float32))
    y_or = orc.linear(W, fmt, x)
    check_close(run_dec(W, fmt, x, act=act), relu(y_or) if act else y_or, f"N={N} KB={KB} M={M} act={act}")


@pytest.mark.parametrize("N,K,M", [(5632, 2048, 16), (5632, 2048, 24), (4112, 1024, 9), (4112, 4160, 20)])
def test_dec_several_tiles_per_workgroup(orc, N, K, M):
    """More row tiles than compute units: 352 tiles (TinyLlama-shaped gate,
    two tiles per workgroup) and 257 tiles (two per workgroup, the last
    workgroup with one), over one round and over several rounds of K
    (4160 = 65 K-blocks: a second round of one K-block), with the column
    refills between tiles and rounds."""
    rng = np.random.default_rng(N + K + M)
    W = (rng.standard_t(4, size=(N, K)) * 0.02).astype(np.float32)
    fmt = rng.integers(0, 5, size=(N, K // 64)).astype(np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    check_close(run_dec(W, fmt, x), orc.linear(W, fmt, x), f"N={N} K={K} M={M}")


@pytest.mark.parametrize("share", [0.03, 0.06])
@pytest.mark.parametrize("N,K,M", [(4096, 4096, 16), (5632, 2048, 16), (4096, 4096, 32)])
def test_dec_load_schemes(orc, share, N, K, M):
    """Both load schemes: a layer whose FP32 blocks are 3% of its blocks
    (under the 4.2% at which a 16-block column holds one with probability
    1/2: the columns skip the pieces no lane needs) and one with 6% (every
    column issues its fixed six loads with the unneeded ones masked), each
    with one step per workgroup (4096 x 4096 at 16 rows), several row tiles
    per workgroup (352 tiles) and two rounds of K (32 rows)."""
    rng = np.random.default_rng(int(share * 1000) + N + M)
    W = (rng.standard_t(4, size=(N, K)) * 0.02).astype(np.float32)
    fmt = np.where(rng.random((N, K // 64)) < share, FP32, INT8).astype(np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    check_close(run_dec(W, fmt, x), orc.linear(W, fmt, x), f"share={share} N={N} K={K} M={M}")
