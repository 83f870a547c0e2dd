"""GPU parity of the input gradient on the matrix cores (ht_linear_backward_data
from 16 rows of dY) against the oracle: dX = dY . W_hat within
1e-3 * max|dX_oracle| (oracle in fp64 from the same fp32 dY).  Covers the
three row-tile sizes (32, 64, 128 rows of dY per workgroup), splits of n
(few output tiles) and no split, ragged M, N and K, every forced format and
mixed plans, unaligned row strides of dY (scalar loads) and of dX (padding
untouched), bitwise determinism, a full 4096 x 4096 layer at 64 rows, and
the Llama-8B q / down projections at 2048 rows checked on sampled rows.
Then the weight gradient on the matrix cores (ht_linear_backward_weight
from 64 rows): ragged shapes, strides, accumulation, determinism and a
4096 x 4096 gradient at 2048 rows in full."""
import numpy as np
import pytest
import torch

from block_planner_amd import api
from block_planner_amd import binding as B
from block_planner_amd import workloads as wl

pytestmark = pytest.mark.gpu
TOL = 1e-3


def dev():
    return torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def check(dx, ref, what):
    dx = np.asarray(dx, np.float64)
    assert np.all(np.isfinite(dx)), what
    err = np.max(np.abs(dx - ref))
    assert err <= TOL * np.max(np.abs(ref)), f"{what}: {err:.3e} vs {np.max(np.abs(ref)):.3e}"


@pytest.mark.parametrize("M", [16, 33, 64, 100, 130, 257])
def test_backward_mfma_mixed_formats(orc, M):
    """200 x 512: 13 row tiles (the last of 8 rows), 8 K-blocks (4 column
    tiles of 128), formats drawn at random per block."""
    rng = np.random.default_rng(170 + M)
    W = (rng.normal(size=(200, 512)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(200, 8)).astype(np.uint8)
    dy = rng.normal(size=(M, 200)).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    dx = api.linear_backward_data(pw, gpu(dy))
    torch.cuda.synchronize()
    check(dx.cpu().numpy(), orc.linear_backward_data(W, fmt, dy), f"M={M}")


@pytest.mark.parametrize("force", [0, 1, 2, 3, 4])
def test_backward_mfma_single_format(orc, force):
    """Every block one format; K = 3 blocks (the second column tile of 128
    holds one K-block), 300 rows of W (19 row tiles)."""
    rng = np.random.default_rng(180 + force)
    W = (rng.standard_t(4, size=(300, 192)) * 0.02).astype(np.float32)
    fmt = orc.plan(W, force=force)
    dy = rng.normal(size=(48, 300)).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    dx = api.linear_backward_data(pw, gpu(dy))
    torch.cuda.synchronize()
    check(dx.cpu().numpy(), orc.linear_backward_data(W, fmt, dy), f"force={force}")


def test_backward_mfma_strides_and_determinism(orc):
    """lddy = N + 3 (not a multiple of 4: dY read one float at a time) and
    lddx = K + 12 (padding untouched); a second call gives the same bits."""
    rng = np.random.default_rng(190)
    N, K, M = 150, 640, 70
    W = (rng.standard_t(4, size=(N, K)) * 0.02).astype(np.float32)
    fmt = orc.plan(W)
    dy = rng.normal(size=(M, N)).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    dys = torch.zeros((M, N + 3), dtype=torch.float32, device=dev())
    dys[:, :N] = gpu(dy)
    dys[:, N:] = 1e30                                 # never read
    dxs = torch.full((M, K + 12), 7.0, dtype=torch.float32, device=dev())
    ws = api.workspace(B.ht_linear_backward_workspace(pw.desc, M), dev())
    B.ht_linear_backward_data(pw.desc, dys[:, :N], dxs[:, :K], ws=ws)
    torch.cuda.synchronize()
    assert torch.all(dxs[:, K:] == 7.0)
    check(dxs[:, :K].cpu().numpy(), orc.linear_backward_data(W, fmt, dy), "strides")
    again = api.linear_backward_data(pw, dys[:, :N].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(again, dxs[:, :K])


def test_backward_mfma_matches_register_path_at_threshold(orc):
    """15 rows take the register path, 16 the matrix cores: both meet the
    bar on the same weight (the rows they share agree to it too)."""
    rng = np.random.default_rng(191)
    W = (rng.standard_t(4, size=(256, 1024)) * 0.02).astype(np.float32)
    fmt = orc.plan(W)
    dy = rng.normal(size=(16, 256)).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    ref = orc.linear_backward_data(W, fmt, dy)
    a = api.linear_backward_data(pw, gpu(dy[:15]))
    b = api.linear_backward_data(pw, gpu(dy))
    torch.cuda.synchronize()
    check(a.cpu().numpy(), ref[:15], "15 rows")
    check(b.cpu().numpy(), ref, "16 rows")


def test_backward_mfma_full_layer_64_rows(orc):
    """The benchmark MLP's 4096 x 4096 layer at 64 rows of dY, every output
    compared (the call splits n: 32 output tiles for 256 compute units)."""
    W = wl.mlp_weight(1)
    fmt = orc.plan(W)
    rng = np.random.default_rng(192)
    dy = rng.normal(size=(64, W.shape[0])).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    dx = api.linear_backward_data(pw, gpu(dy))
    torch.cuda.synchronize()
    check(dx.cpu().numpy(), orc.linear_backward_data(W, fmt, dy), "mlp4096 M=64")


@pytest.mark.parametrize("name", ["q", "down"])
def test_backward_mfma_llama_2048_rows_sampled(orc, name):
    """Llama-8B q (4096 x 4096) and down (4096 x 14336) at 2048 rows of dY
    (no split: the output tiles fill the chip); 24 sampled rows of dX against
    the oracle on those rows of dY (rows of dX depend only on their row of
    dY)."""
    shp = [s for s in wl.llama8b_shapes() if s.name == name][0]
    W = wl.llama8b_weight(0, shp)
    fmt = orc.plan(W)
    rng = np.random.default_rng(193)
    M = 2048
    dy = rng.normal(size=(M, shp.n)).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    dx = api.linear_backward_data(pw, gpu(dy))
    torch.cuda.synchronize()
    rows = np.sort(np.concatenate([[0, 127, 128, M - 1], rng.choice(M, size=20, replace=False)]))
    got = dx[torch.from_numpy(rows).to(dev())].cpu().numpy()
    check(got, orc.linear_backward_data(W, fmt, dy[rows]), f"{name} M=2048 sampled")


# ---------------------------------------------------------------------------
# The STE weight gradient dW = dY^T . x on the matrix cores (from 64 rows)
# ---------------------------------------------------------------------------
def _dw_case(M, N, K, seed, lddy=None, ldx=None):
    rng = np.random.default_rng(seed)
    dy = rng.normal(size=(M, lddy or N)).astype(np.float32)
    xb = wl.to_bf16_bits(rng.normal(size=(M, ldx or K)).astype(np.float32))
    return dy, xb


@pytest.mark.parametrize("M,N,K", [(63, 64, 64), (64, 200, 192), (100, 130, 1028), (257, 300, 512),
                                   (65, 129, 132), (130, 77, 256)])
def test_weight_grad_mfma_matches_oracle(orc, M, N, K):
    """Ragged M (steps of 64 rows), N and K (tiles of 128), K not a multiple
    of 128; 63 rows (the vector path) beside 64 and more; odd N (dY read one
    float at a time, the last column alone)."""
    dy, xb = _dw_case(M, N, K, 270 + M)
    dw = torch.full((N, K), float("nan"), device=dev())
    B.ht_linear_backward_weight(gpu(dy), gpu(xb.view(np.int16)), dw)
    torch.cuda.synchronize()
    check(dw.cpu().numpy(), orc.linear_backward_weight(dy, xb), f"dW M={M} N={N} K={K}")


@pytest.mark.parametrize("lddy", [96, 83])
def test_weight_grad_mfma_accumulate_strides_determinism(orc, lddy):
    """lddy 96 (float4 reads) and 83 (one float at a time), ldx 260, lddw
    264: accumulation into dw, columns past K untouched, two calls give the
    same bits."""
    M, N, K = 70, 80, 256
    dy, xb = _dw_case(M, N, K, 280, lddy=lddy, ldx=260)
    ref = orc.linear_backward_weight(dy[:, :N], xb[:, :K])
    base = torch.randn(N, 264, device=dev())
    dw = base.clone()
    args = dict(M=M, N=N, K=K, lddy=lddy, ldx=260, lddw=264)
    B.ht_linear_backward_weight(gpu(dy), gpu(xb.view(np.int16)), dw, accumulate=True, **args)
    torch.cuda.synchronize()
    got = dw.cpu().numpy().astype(np.float64)
    check(got[:, :K] - base.cpu().numpy()[:, :K], ref, "accumulate")
    assert torch.equal(dw[:, K:], base[:, K:])
    d1 = torch.empty(N, 264, device=dev())
    d2 = torch.empty(N, 264, device=dev())
    for d in (d1, d2):
        B.ht_linear_backward_weight(gpu(dy), gpu(xb.view(np.int16)), d, **args)
    torch.cuda.synchronize()
    assert torch.equal(d1[:, :K], d2[:, :K])


def test_weight_grad_mfma_full_size_2048_rows(orc):
    """A 4096 x 4096 weight gradient at 2048 rows, whole output against
    fp64."""
    dy, xb = _dw_case(2048, 4096, 4096, 290)
    dw = torch.empty(4096, 4096, device=dev())
    B.ht_linear_backward_weight(gpu(dy), gpu(xb.view(np.int16)), dw)
    torch.cuda.synchronize()
    check(dw.cpu().numpy(), orc.linear_backward_weight(dy, xb), "dW 4096x4096 M=2048")
