"""GPU parity of the input gradient (ht_linear_backward_data) against the
oracle: dX = dY . W_hat within 1e-3 * max|dX_oracle| (oracle in fp64 from the
same fp32 dY), over mixed and forced formats, ragged N, several launches of
4 rows, row strides, full-size Llama-shaped weights, and bitwise determinism;
and the STE weight gradient (ht_linear_backward_weight) against the oracle's
dY^T . x."""
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


@pytest.mark.parametrize("M", [1, 3, 4, 5, 9])
def test_backward_mixed_formats(orc, M):
    rng = np.random.default_rng(70 + M)
    W = (rng.normal(size=(200, 512)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(200, 8)).astype(np.uint8)
    dy = rng.normal(size=(M, 200)).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    dx = api.linear_backward_data(pw, gpu(dy))
    torch.cuda.synchronize()
    check(dx.cpu().numpy(), orc.linear_backward_data(W, fmt, dy), f"M={M}")


@pytest.mark.parametrize("force", [0, 1, 2, 3, 4])
def test_backward_single_format(orc, force):
    W = wl.small_weight(seed=5)
    fmt = orc.plan(W, force=force)
    rng = np.random.default_rng(80 + force)
    dy = rng.normal(size=(2, W.shape[0])).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    dx = api.linear_backward_data(pw, gpu(dy))
    torch.cuda.synchronize()
    check(dx.cpu().numpy(), orc.linear_backward_data(W, fmt, dy), f"force={force}")


def test_backward_strides_and_determinism(orc):
    rng = np.random.default_rng(90)
    W = (rng.standard_t(4, size=(72, 1024)) * 0.02).astype(np.float32)
    fmt = orc.plan(W)
    dy = rng.normal(size=(6, 72)).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    dys = torch.zeros((6, 72 + 20), dtype=torch.float32, device=dev())
    dys[:, :72] = gpu(dy)
    dxs = torch.full((6, 1024 + 12), 7.0, dtype=torch.float32, device=dev())
    ws = api.workspace(B.ht_linear_backward_workspace(pw.desc, 6), dev())
    B.ht_linear_backward_data(pw.desc, dys[:, :72], dxs[:, :1024], ws=ws)
    torch.cuda.synchronize()
    assert torch.all(dxs[:, 1024:] == 7.0)
    check(dxs[:, :1024].cpu().numpy(), orc.linear_backward_data(W, fmt, dy), "strides")
    again = api.linear_backward_data(pw, dys[:, :72].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(again, dxs[:, :1024])


@pytest.mark.parametrize("name,M", [("q", 1), ("down", 2), ("k", 4)])
def test_backward_full_size(orc, name, M):
    shp = [s for s in wl.llama8b_shapes() if s.name == name][0]
    W = wl.llama8b_weight(0, shp)
    fmt = orc.plan(W)
    rng = np.random.default_rng(91)
    dy = rng.normal(size=(M, shp.n)).astype(np.float32)
    pw = api.pack(gpu(W), gpu(fmt))
    dx = api.linear_backward_data(pw, gpu(dy))
    torch.cuda.synchronize()
    check(dx.cpu().numpy(), orc.linear_backward_data(W, fmt, dy), f"{name} M={M}")


def test_backward_row_tile_restriction():
    W = wl.small_weight()
    fmt = torch.zeros((256, 4), dtype=torch.uint8, device=dev())
    pw = api.pack(gpu(W), fmt, row_tile=8)
    with pytest.raises(B.HTError):
        B.ht_linear_backward_workspace(pw.desc, 1)


# ---------------------------------------------------------------------------
# STE weight gradient dW = dY^T . x
# ---------------------------------------------------------------------------
def _dw_case(M, N, K, seed, lddy=None, ldx=None, lddw=None):
    rng = np.random.default_rng(seed)
    dy = rng.normal(size=(M, lddy or N)).astype(np.float32)
    xb = wl.to_bf16_bits(rng.normal(size=(M, ldx or K)).astype(np.float32))
    return dy, xb


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (5, 200, 192), (33, 96, 320), (3, 17, 1028)])
def test_weight_grad_matches_oracle(orc, M, N, K):
    dy, xb = _dw_case(M, N, K, 70 + M)
    dw = torch.full((N, K), float("nan"), device=dev())
    B.ht_linear_backward_weight(gpu(dy), gpu(xb.view(np.int16)), dw)
    torch.cuda.synchronize()
    check(dw.cpu().numpy(), orc.linear_backward_weight(dy, xb), f"dW M={M} N={N} K={K}")


def test_weight_grad_accumulate_strides_determinism_and_empty(orc):
    M, N, K = 7, 80, 256
    dy, xb = _dw_case(M, N, K, 80, lddy=96, ldx=260)
    ref = orc.linear_backward_weight(dy[:, :N], xb[:, :K])
    base = torch.randn(N, 264, device=dev())
    dw = base.clone()
    args = dict(M=M, N=N, K=K, lddy=96, ldx=260, lddw=264)
    B.ht_linear_backward_weight(gpu(dy), gpu(xb.view(np.int16)), dw, accumulate=True, **args)
    torch.cuda.synchronize()
    got = dw.cpu().numpy().astype(np.float64)
    check(got[:, :K] - base.cpu().numpy()[:, :K], ref, "accumulate")
    assert torch.equal(dw[:, K:], base[:, K:])                           # columns past K untouched
    d1 = torch.empty(N, 264, device=dev())
    d2 = torch.empty(N, 264, device=dev())
    for d in (d1, d2):
        B.ht_linear_backward_weight(gpu(dy), gpu(xb.view(np.int16)), d, **args)
    torch.cuda.synchronize()
    assert torch.equal(d1[:, :K], d2[:, :K])
    z = torch.full((N, K), 5.0, device=dev())                            # M = 0: zeros, or left as is
    B.ht_linear_backward_weight(gpu(dy), gpu(xb.view(np.int16)), z, M=0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z).item() == 0


def test_weight_grad_full_size(orc):
    """A 4096 x 4096 layer at 32 rows of dY, whole output against fp64."""
    dy, xb = _dw_case(32, 4096, 4096, 90)
    dw = torch.empty(4096, 4096, device=dev())
    B.ht_linear_backward_weight(gpu(dy), gpu(xb.view(np.int16)), dw)
    torch.cuda.synchronize()
    check(dw.cpu().numpy(), orc.linear_backward_weight(dy, xb), "dW 4096x4096 M=32")
