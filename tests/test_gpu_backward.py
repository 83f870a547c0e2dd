"""GPU parity of the input gradient (ht_linear_backward_data) against the
oracle: dX = dY . W_hat within 1e-3 * max|dX_oracle| (oracle in fp64 from the
same fp32 dY), over mixed and forced formats, ragged N, several launches of
4 rows, row strides, full-size Llama-shaped weights, and bitwise determinism."""
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
