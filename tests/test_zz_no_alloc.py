"""ht_linear_forward_noalloc, the workspace-free variant of ht_linear_forward
for callers that cannot allocate device memory: on every path whose kernels
use a workspace (K-split partial sums, the int8 path's encoded x), two calls
in a row on the library's fixed array, the second with fewer rows, each
bitwise equal to ht_linear_forward with a workspace of its own on the same
path (the same kernels), and the first within the bar of the oracle."""
import numpy as np
import pytest
import torch

from block_planner_amd import api
from block_planner_amd import binding as B
from block_planner_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 1e-3

CASES = [
    # name, N, K, path, forced format (-1: plan), rows of the first and second call
    ("register path, K split", 512, 14336, B.HT_PATH_GEMV, -1, 8, 3),
    ("MFMA decode path, K split over few row tiles", 256, 4096, B.HT_PATH_GEMV_MFMA, -1, 32, 5),
    ("MFMA path, K split", 1024, 4096, B.HT_PATH_GEMM, -1, 256, 40),
    ("int8 path, all-INT8 weight", 512, 4096, B.HT_PATH_GEMM_I8, 1, 256, 64),
    ("int8 path next to the MFMA path", 512, 4096, B.HT_PATH_GEMM_I8, -1, 128, 48),
]


def dev():
    return torch.device("cuda:0")


@pytest.mark.parametrize("name,N,K,path,force,M1,M2", CASES)
def test_noalloc_matches_workspace_call(orc, name, N, K, path, force, M1, M2):
    rng = np.random.default_rng(N + K + path)
    W = (rng.standard_t(4, size=(N, K)) * 0.02).astype(np.float32)
    if path == B.HT_PATH_GEMM_I8 and force < 0:
        # rows 0..255 on the INT8 grid (every block reaches 127; too spread for INT4): that 256-row
        # tile is all INT8 and runs on the int8 kernel, the rest on the MFMA path
        k = np.clip(np.round(rng.normal(0.0, 30.0, size=(256, K))), -127, 127)
        k[:, ::64] = 127
        W[:256] = (k * 2.0 ** -10).astype(np.float32)
    Wg = torch.from_numpy(W).to(dev())
    fmt = api.plan(Wg, force_format=force)
    pw = api.pack(Wg, fmt)
    assert B.ht_linear_workspace(pw.desc, M1, path) > 0, name   # the call does use a workspace
    for call, M in enumerate((M1, M2)):
        xb = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
        x = torch.from_numpy(xb.view(np.int16)).to(dev()).view(torch.bfloat16)
        y_ref = api.linear(pw, x, path=path)
        y = torch.full((M, N), 7.0, dtype=torch.float32, device=dev())
        B.ht_linear_forward_noalloc(pw.desc, x, y, path=path)
        torch.cuda.synchronize()
        print(f"{name}: call {call}, M = {M}", flush=True)
        assert torch.equal(y, y_ref), f"{name}: call {call} differs from ht_linear_forward"
        if call == 0:
            y_or = orc.linear(W, fmt.cpu().numpy(), xb)
            err = float(np.max(np.abs(y.cpu().numpy() - y_or)))
            assert err <= TOL * float(np.max(np.abs(y_or))), name


def test_noalloc_refuses_what_exceeds_the_array():
    """A call needing more workspace than the fixed array reports HT_ESMALL
    and launches nothing (the output keeps its contents)."""
    N, K, M = 512, 14336, 2048
    Wg = (torch.randn(N, K, device=dev()) * 0.02)
    fmt = api.plan(Wg, force_format=1)
    pw = api.pack(Wg, fmt)
    need = B.ht_linear_workspace(pw.desc, M, B.HT_PATH_GEMM_I8)
    assert need > (32 << 20)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=dev())
    y = torch.full((M, N), 7.0, dtype=torch.float32, device=dev())
    with pytest.raises(B.HTError) as e:
        B.ht_linear_forward_noalloc(pw.desc, x, y, path=B.HT_PATH_GEMM_I8)
    assert e.value.code == 4
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
