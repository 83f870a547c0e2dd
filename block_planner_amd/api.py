"""Convenience layer over the C ABI: allocates device buffers with torch and
calls the ``ht_*`` entry points.  No arithmetic of the method happens here.

    fmt = plan(W)                      # uint8 [N, K/64] on the GPU
    pw  = pack(W, fmt)                 # PackedLinear (owns its buffer)
    y   = linear(pw, x_bf16)           # fp32 [M, N]
    y   = mlp([pw0, pw1, ...], x_bf16) # Linear + ReLU per layer
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


@dataclass
class PackedLinear:
    buf: torch.Tensor            # uint8 device buffer (owned)
    desc: B.PackedWeight
    counts: list

    @property
    def N(self) -> int:
        return int(self.desc.N)

    @property
    def K(self) -> int:
        return int(self.desc.K)

    @property
    def nbytes(self) -> int:
        return int(self.desc.bytes)


def plan_params(eps_int4=0.08, eps_int8=0.01, eps_bf16=0.0, eps_fp16=0.0, prefer_bf16=True,
                force_format=-1) -> B.PlanParams:
    p = B.PlanParams()
    p.eps_int4, p.eps_int8, p.eps_bf16, p.eps_fp16 = eps_int4, eps_int8, eps_bf16, eps_fp16
    p.prefer_bf16 = 1 if prefer_bf16 else 0
    p.force_format = force_format
    return p


def plan(W: torch.Tensor, stream=None, **params) -> torch.Tensor:
    N, K = W.shape
    fmt = torch.empty((N, K // 64), dtype=torch.uint8, device=W.device)
    B.ht_plan(W, fmt, plan_params(**params), stream=stream)
    return fmt


def counts(fmt: torch.Tensor, stream=None) -> list:
    c = torch.empty(5, dtype=torch.int64, device=fmt.device)
    B.ht_plan_counts(fmt, c, stream=stream)
    return [int(v) for v in c.cpu()]


def _aligned_empty(nbytes: int, device, align: int = 256) -> torch.Tensor:
    raw = torch.empty(nbytes + align, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % align
    return raw[off:off + nbytes]


def pack(W: torch.Tensor, fmt: torch.Tensor, row_tile: int = 16, stream=None, cnt=None) -> PackedLinear:
    N, K = W.shape
    cnt = counts(fmt, stream=stream) if cnt is None else cnt
    nbytes = B.ht_pack_bytes(N, K, row_tile, cnt)
    buf = _aligned_empty(nbytes, W.device)
    desc = B.ht_pack(W, fmt, row_tile, cnt, buf, stream=stream)
    return PackedLinear(buf=buf, desc=desc, counts=cnt)


@dataclass
class RefreshState:
    """Buffers of ht_refresh for one weight shape, allocated once: the packed
    buffer at its upper bound, the format map, the device counts and the
    initialised workspace."""
    N: int
    K: int
    row_tile: int
    buf: torch.Tensor
    fmt: torch.Tensor
    counts: torch.Tensor
    ws: torch.Tensor


def refresh_state(N: int, K: int, row_tile: int, device, stream=None) -> RefreshState:
    buf_bytes, ws_bytes = B.ht_refresh_bytes(N, K, row_tile)
    ws = _aligned_empty(ws_bytes, device)
    B.ht_workspace_init(ws, stream=stream)
    return RefreshState(N, K, row_tile, _aligned_empty(buf_bytes, device),
                        torch.empty((N, K // 64), dtype=torch.uint8, device=device),
                        torch.empty(5, dtype=torch.int64, device=device), ws)


def refresh(W: torch.Tensor, st: RefreshState, stream=None, **params) -> PackedLinear:
    """Re-plan and re-pack W into st.buf in one pass (ht_refresh), then
    build the descriptor from the counts (one 40-byte copy to the host).
    The previous packed weight of st is overwritten."""
    B.ht_refresh(W, st.fmt, st.buf, st.counts, st.ws, plan_params(**params), row_tile=st.row_tile, stream=stream)
    cnt = [int(v) for v in st.counts.cpu()]
    if int(st.ws[8:12].view(torch.int32).item()) != 0:
        raise RuntimeError("ht_refresh: a wait between workgroups expired (not all workgroups were resident); "
                           "the refreshed buffer is invalid")
    desc = B.ht_refresh_desc(st.N, st.K, st.row_tile, cnt, st.buf)
    return PackedLinear(buf=st.buf[:int(desc.bytes)], desc=desc, counts=cnt)


def workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return _aligned_empty(nbytes, device)


def linear(pw: PackedLinear, x: torch.Tensor, act: int = B.HT_ACT_NONE, out: torch.Tensor | None = None,
           ws: torch.Tensor | None = None, path: int = B.HT_PATH_AUTO, stream=None) -> torch.Tensor:
    M = x.shape[0]
    y = torch.empty((M, pw.N), dtype=torch.float32, device=x.device) if out is None else out
    if ws is None:
        ws = workspace(B.ht_linear_workspace(pw.desc, M, path), x.device)
    B.ht_linear_forward(pw.desc, x, y, act=act, path=path, ws=ws, stream=stream)
    return y


def linear_backward_data(pw: PackedLinear, dy: torch.Tensor, out: torch.Tensor | None = None,
                         ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """dX = dY . W_hat (fp32 dY [M, N] -> fp32 dX [M, K])."""
    M = dy.shape[0]
    dx = torch.empty((M, pw.K), dtype=torch.float32, device=dy.device) if out is None else out
    if ws is None:
        ws = workspace(B.ht_linear_backward_workspace(pw.desc, M), dy.device)
    B.ht_linear_backward_data(pw.desc, dy, dx, ws=ws, stream=stream)
    return dx


def linear_backward_weight(dy: torch.Tensor, x_bf16: torch.Tensor, out: torch.Tensor | None = None,
                           accumulate: bool = False, stream=None) -> torch.Tensor:
    """dW = dY^T . x (STE gradient of the fp32 master; fp32 [N, K]); with
    accumulate the product is added to `out`."""
    M, N = dy.shape
    K = x_bf16.shape[1]
    dw = torch.empty((N, K), dtype=torch.float32, device=dy.device) if out is None else out
    B.ht_linear_backward_weight(dy, x_bf16, dw, accumulate=accumulate, stream=stream)
    return dw


def mlp_workspace(layers: list, M: int, device, stream=None) -> torch.Tensor:
    """An initialised workspace for mlp() over these layers at batch M."""
    ws = workspace(B.ht_mlp_workspace([pw.desc for pw in layers], M), device)
    B.ht_workspace_init(ws, stream=stream)
    return ws


def mlp(layers: list, x: torch.Tensor, dump: bool = False, out: torch.Tensor | None = None,
        ws: torch.Tensor | None = None, path: int = B.HT_PATH_AUTO, stream=None):
    M = x.shape[0]
    descs = [pw.desc for pw in layers]
    y = torch.empty((M, layers[-1].N), dtype=torch.float32, device=x.device) if out is None else out
    if ws is None:
        ws = mlp_workspace(layers, M, x.device, stream=stream)
    act_dump = None
    if dump:
        tot = sum(M * pw.N for pw in layers[:-1])
        act_dump = torch.empty(max(tot, 8), dtype=torch.bfloat16, device=x.device)
    B.ht_mlp_forward(descs, x, y, act_dump=act_dump, path=path, ws=ws, stream=stream)
    if dump:
        slabs, off = [], 0
        for pw in layers[:-1]:
            slabs.append(act_dump[off:off + M * pw.N].view(M, pw.N))
            off += M * pw.N
        return y, slabs
    return y
