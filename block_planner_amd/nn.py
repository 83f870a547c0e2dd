"""PyTorch modules over the C ABI: HyperLinear, scan_model,
wrap_model_with_hypertensor and save/load of packed models.

Follows the user calls of the HyperTensor 1.0.1 page ("Usage Example":
HyperLinear layers with ReLU; "Convert model": scan_model, then
wrap_model_with_hypertensor with inference_only; "Key Features": a drop-in
replacement for nn.Linear, inference-only mode without FP32 master weights,
serializable quantized models and plans).  Every number is computed by the
library's kernels (ht_plan, ht_pack, ht_linear_forward); this module only
allocates, reshapes and casts the activations to bfloat16.

Scope, as built:
  * Linear layers without bias whose in_features is a multiple of 64 and
    whose weight is fp32 on a GPU are converted; the others are left as they
    are and reported in the plan's "skipped" list with the reason.
  * The output is fp32 (the path's accumulation type); the input is cast to
    bfloat16 (round to nearest even) as the path defines.
  * Backward: dX = dY . W_hat by the library's backward kernel
    (ht_linear_backward_data), in fp32, the rounding of x to bfloat16 passed
    straight through; and, when the module keeps a trainable fp32 master
    weight, its straight-through gradient dW = dY^T . x_bf16
    (ht_linear_backward_weight).  An optimizer updates the master; the packed
    buffers follow it at the next refresh (refresh_every) or pack().
  * The planner modes named on the page (LOWEST ... BEST) have no definition
    there; only the per-block rule is accepted (option None or "PER_BLOCK").
  * refresh_every > 0 with a master weight re-plans and re-packs every that
    many forward calls (the page's refresh cadence) with the fused single
    pass ht_refresh, into buffers allocated once.
"""
from __future__ import annotations

import json
import math

import torch

from . import api
from . import binding as B

_DESC_FIELDS = ("N", "K", "row_tile", "n_tiles", "off_kbidx", "bytes", "layout_version")


def _eps(eps_int4=0.08, eps_int8=0.01, eps_bf16=0.0, eps_fp16=0.0, prefer_bf16=True) -> dict:
    return dict(eps_int4=float(eps_int4), eps_int8=float(eps_int8), eps_bf16=float(eps_bf16),
                eps_fp16=float(eps_fp16), prefer_bf16=bool(prefer_bf16))


def _check_row_tile(row_tile: int, inference_only: bool) -> None:
    if int(row_tile) not in (1, 2, 4, 8, 16):
        raise ValueError("row_tile must be one of 1, 2, 4, 8, 16")
    if not inference_only and int(row_tile) != 16:
        # the input-gradient kernel reads 16-row tiles; refuse now rather than
        # in the first backward pass
        raise ValueError("a trainable HyperLinear needs row_tile 16 (the backward kernels' tile)")


class _PackedLinearFn(torch.autograd.Function):
    """y = bf16(x) . W_hat^T forward; backward dX = dY . W_hat and the STE
    gradient of the master, dW = dY^T . bf16(x) (fp32)."""

    @staticmethod
    def forward(ctx, x2: torch.Tensor, weight, packed: api.PackedLinear) -> torch.Tensor:
        xb = x2.to(torch.bfloat16).contiguous()
        ctx.packed = packed
        if ctx.needs_input_grad[1]:
            ctx.save_for_backward(xb)
        return api.linear(packed, xb)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        dy = dy.to(torch.float32).contiguous()
        dx = api.linear_backward_data(ctx.packed, dy) if ctx.needs_input_grad[0] else None
        dw = api.linear_backward_weight(dy, ctx.saved_tensors[0]) if ctx.needs_input_grad[1] else None
        return dx, dw, None


class HyperLinear(torch.nn.Module):
    """y = x . W_hat^T on the packed execution buffers of W (no bias).

    Built from a master weight (an nn.Parameter, fp32, on a GPU), planned and
    packed on the first forward call (or by ``pack()``); with
    ``inference_only`` the master weight is dropped once packed."""

    def __init__(self, in_features: int, out_features: int, bias: bool = False, refresh_every: int = 0,
                 prefer_bf16: bool = True, eps_int4: float = 0.08, eps_int8: float = 0.01, eps_bf16: float = 0.0,
                 eps_fp16: float = 0.0, row_tile: int = 16, inference_only: bool = False, device=None):
        super().__init__()
        if bias:
            raise ValueError("HyperLinear has no bias (the per-block linear is y = x . W_hat^T)")
        if in_features % 64:
            raise ValueError("in_features must be a multiple of 64 (64-wide K-blocks)")
        _check_row_tile(row_tile, inference_only)
        self.in_features, self.out_features = int(in_features), int(out_features)
        self.refresh_every = int(refresh_every)
        self.row_tile = int(row_tile)
        self.inference_only = bool(inference_only)
        self.eps = _eps(eps_int4, eps_int8, eps_bf16, eps_fp16, prefer_bf16)
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        w = torch.empty(out_features, in_features, dtype=torch.float32, device=dev)
        torch.nn.init.kaiming_uniform_(w, a=math.sqrt(5))      # nn.Linear's initialisation
        self.weight = torch.nn.Parameter(w, requires_grad=not self.inference_only)
        self.packed: api.PackedLinear | None = None
        self.fmt: torch.Tensor | None = None
        self._rs: api.RefreshState | None = None
        self._calls = 0

    # -- construction from existing layers / buffers --------------------------
    @classmethod
    def from_linear(cls, lin: torch.nn.Linear, fmt: torch.Tensor | None = None, inference_only: bool = True,
                    row_tile: int = 16, **eps) -> "HyperLinear":
        _check_row_tile(row_tile, inference_only)
        m = cls.__new__(cls)
        torch.nn.Module.__init__(m)
        m.in_features, m.out_features = lin.in_features, lin.out_features
        m.refresh_every, m.row_tile, m.inference_only = 0, int(row_tile), bool(inference_only)
        m.eps = _eps(**eps)
        m.weight = torch.nn.Parameter(lin.weight.detach().to(torch.float32).contiguous(),
                                      requires_grad=not m.inference_only)
        m.packed, m.fmt, m._rs, m._calls = None, None, None, 0
        m.pack(fmt)
        return m

    @classmethod
    def from_packed(cls, packed: api.PackedLinear, fmt: torch.Tensor | None = None) -> "HyperLinear":
        m = cls.__new__(cls)
        torch.nn.Module.__init__(m)
        m.in_features, m.out_features = packed.K, packed.N
        m.refresh_every, m.row_tile, m.inference_only = 0, int(packed.desc.row_tile), True
        m.eps = _eps()
        m.weight = None
        m.packed, m.fmt, m._rs, m._calls = packed, fmt, None, 0
        return m

    # -- planning and packing ---------------------------------------------------
    def pack(self, fmt: torch.Tensor | None = None) -> None:
        """Plan (unless a format map is given) and pack the master weight.

        A module that refreshes (refresh_every > 0, not inference-only)
        re-plans and re-packs with the fused single pass (ht_refresh) into
        buffers allocated on its first pack and reused afterwards; the
        packed buffer is overwritten in place, so a backward pass must run
        before the module's next refresh."""
        if self.weight is None:
            raise RuntimeError("no master weight to pack (inference-only module)")
        W = self.weight.detach()
        if fmt is None and self.refresh_every > 0 and not self.inference_only:
            if self._rs is None:
                self._rs = api.refresh_state(self.out_features, self.in_features, self.row_tile, W.device)
            self.packed = api.refresh(W.contiguous(), self._rs, **self.eps)
            self.fmt = self._rs.fmt
            return
        self.fmt = api.plan(W, **self.eps) if fmt is None else fmt.to(device=W.device, dtype=torch.uint8)
        self.packed = api.pack(W, self.fmt, row_tile=self.row_tile)
        if self.inference_only:
            self.weight = None

    def memory_bytes(self) -> dict:
        """Device bytes held: the packed buffer and, unless inference-only,
        the fp32 master weight."""
        packed = self.packed.nbytes if self.packed is not None else 0
        master = self.weight.numel() * 4 if self.weight is not None else 0
        held = int(self._rs.buf.numel()) if self._rs is not None else packed   # the refresh buffer's full size
        return {"packed": packed, "master_fp32": master, "total": held + master}

    # -- forward -----------------------------------------------------------------
    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if self.packed is None or (self.refresh_every > 0 and self.weight is not None and self._calls > 0
                                   and self._calls % self.refresh_every == 0):
            self.pack()
        self._calls += 1
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected {self.in_features} input features, got {x.shape[-1]}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if x2.shape[0] == 0:
            return torch.empty(*lead, self.out_features, dtype=torch.float32, device=x.device)
        w_grad = self.weight is not None and self.weight.requires_grad
        if torch.is_grad_enabled() and (x2.requires_grad or w_grad):
            y = _PackedLinearFn.apply(x2, self.weight if w_grad else None, self.packed)
        else:
            y = api.linear(self.packed, x2.to(torch.bfloat16).contiguous())
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        mix = ""
        if self.packed is not None:
            tot = sum(self.packed.counts) or 1
            mix = ", mix=" + "/".join(f"{c / tot:.3f}" for c in self.packed.counts)
        return f"in_features={self.in_features}, out_features={self.out_features}{mix}"


# -----------------------------------------------------------------------------
# Model conversion
# -----------------------------------------------------------------------------
def _linear_ok(mod: torch.nn.Linear) -> str | None:
    if mod.bias is not None:
        return "has a bias"
    if mod.in_features % 64:
        return "in_features is not a multiple of 64"
    if not mod.weight.is_cuda:
        return "weight is not on a GPU"
    if mod.weight.dtype != torch.float32:
        return "weight is not fp32"
    return None


def scan_model(model: torch.nn.Module, eps_fp16: float = 0.0, eps_bf16: float = 0.0, prefer_bf16: bool = True,
               eps_int4: float = 0.08, eps_int8: float = 0.01) -> dict:
    """Plan every convertible nn.Linear of `model` ("Convert model":
    scan_model).  Returns {"layers": {name: {"fmt": uint8 [N, K/64] on the
    GPU, "counts": [5]}}, "skipped": {name: reason}, "eps": {...}}."""
    eps = _eps(eps_int4, eps_int8, eps_bf16, eps_fp16, prefer_bf16)
    layers, skipped = {}, {}
    for name, mod in model.named_modules():
        if not isinstance(mod, torch.nn.Linear):
            continue
        why = _linear_ok(mod)
        if why:
            skipped[name] = why
            continue
        fmt = api.plan(mod.weight.detach().contiguous(), **eps)
        layers[name] = {"fmt": fmt, "counts": api.counts(fmt)}
    return {"layers": layers, "skipped": skipped, "eps": eps}


def _set_child(model: torch.nn.Module, name: str, new: torch.nn.Module) -> None:
    parent = model
    parts = name.split(".")
    for p in parts[:-1]:
        parent = getattr(parent, p)
    setattr(parent, parts[-1], new)


def wrap_model_with_hypertensor(model: torch.nn.Module, plan: dict, option=None, inference_only: bool = True,
                                row_tile: int = 16) -> torch.nn.Module:
    """Replace every planned nn.Linear of `model` by a HyperLinear packed
    from its plan ("Convert model": wrap_model_with_hypertensor).  In place;
    returns `model`."""
    if option not in (None, "PER_BLOCK"):
        raise ValueError(f"planner option {option!r} is not defined; only the per-block rule (None / 'PER_BLOCK')")
    mods = dict(model.named_modules())
    for name, entry in plan["layers"].items():
        lin = mods.get(name)
        if not isinstance(lin, torch.nn.Linear):
            raise KeyError(f"{name!r} is not an nn.Linear of this model")
        _set_child(model, name, HyperLinear.from_linear(lin, entry["fmt"], inference_only=inference_only,
                                                        row_tile=row_tile, **plan.get("eps", {})))
    return model


# -----------------------------------------------------------------------------
# Serialization (safetensors: packed buffers as uint8 tensors, descriptors and
# format maps alongside; loading executes nothing from the file)
# -----------------------------------------------------------------------------
def save_hypertensor(model: torch.nn.Module, path: str) -> None:
    from safetensors.torch import save_file

    tensors, meta = {}, {}
    for name, mod in model.named_modules():
        if isinstance(mod, HyperLinear) and mod.packed is not None:
            d = mod.packed.desc
            tensors[f"{name}.packed"] = mod.packed.buf.detach().cpu().contiguous()
            if mod.fmt is not None:
                tensors[f"{name}.fmt"] = mod.fmt.detach().cpu().contiguous()
            meta[name] = {**{f: int(getattr(d, f)) for f in _DESC_FIELDS},
                          "counts": [int(c) for c in d.counts], "off_ids": [int(v) for v in d.off_ids],
                          "off_scale": [int(v) for v in d.off_scale],
                          "off_payload": [int(v) for v in d.off_payload]}
    save_file(tensors, path, metadata={"hypertensor_layers": json.dumps(meta)})


def read_hypertensor(path: str) -> list:
    """The packed layers of a file written by save_hypertensor, validated in
    host memory before anything reaches a device: each descriptor must match
    the layout of its (N, K, row tile, counts) and each buffer's block index
    must describe a format map (ht_check_packed), equal to the stored map
    when one is stored.  Returns [(name, host uint8 tensor, PackedWeight with
    base unset, counts, host fmt uint8 [N, K/64] or None)]; raises ValueError
    for a file that fails."""
    import numpy as np
    from safetensors import safe_open

    out = []
    with safe_open(path, framework="pt") as f:
        meta = json.loads(f.metadata()["hypertensor_layers"])
        keys = set(f.keys())
        for name, m in meta.items():
            try:
                host = f.get_tensor(f"{name}.packed")
                if host.dtype != torch.uint8 or host.dim() != 1:
                    raise ValueError("packed buffer is not a 1-D uint8 tensor")
                d = B.PackedWeight()
                for fld in _DESC_FIELDS:
                    setattr(d, fld, int(m[fld]))
                for arr, key, n in ((d.counts, "counts", 5), (d.off_ids, "off_ids", 5),
                                    (d.off_scale, "off_scale", 2), (d.off_payload, "off_payload", 5)):
                    vals = [int(v) for v in m[key]]
                    if len(vals) != n:
                        raise ValueError(f"{key} has {len(vals)} entries, expected {n}")
                    for i, v in enumerate(vals):
                        arr[i] = v
                if host.numel() != int(d.bytes):
                    raise ValueError(f"buffer holds {host.numel()} bytes, descriptor says {int(d.bytes)}")
                hb = host.numpy()
                fmt_idx = np.zeros((int(d.N), int(d.K) // 64), np.uint8)
                B.ht_check_packed(d, hb, fmt_idx)
                fmt = None
                if f"{name}.fmt" in keys:
                    fmt = f.get_tensor(f"{name}.fmt")
                    if tuple(fmt.shape) != fmt_idx.shape or not np.array_equal(fmt.numpy(), fmt_idx):
                        raise ValueError("stored format map differs from the buffer's block index")
            except (B.HTError, KeyError, TypeError, OverflowError) as e:
                raise ValueError(f"{path}: layer {name!r} is not a valid packed weight: {e}") from e
            except ValueError as e:
                raise ValueError(f"{path}: layer {name!r} is not a valid packed weight: {e}") from e
            out.append((name, host, d, [int(c) for c in m["counts"]], fmt))
    return out


def load_hypertensor(model: torch.nn.Module, path: str, device=None) -> torch.nn.Module:
    """Put the packed layers saved by save_hypertensor into `model` (whose
    modules of those names are replaced by inference-only HyperLinear).  Every
    layer is validated on the host first (read_hypertensor); the packed bytes
    are then copied to a 256-byte aligned device buffer."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    for name, host, d, counts, fmt in read_hypertensor(path):
        buf = api._aligned_empty(host.numel(), dev)
        buf.copy_(host)
        d.base = buf.data_ptr()
        fmt_d = fmt.to(dev) if fmt is not None else None
        _set_child(model, name, HyperLinear.from_packed(api.PackedLinear(buf, d, counts), fmt_d))
    return model
