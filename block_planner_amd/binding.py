"""ctypes binding of ``libht.so`` -- argument marshalling only.

Every function named ``ht_*`` here forwards to the C entry point of the same
name declared in ``include/ht.h``; tensors are passed as raw device pointers
(``tensor.data_ptr()``) and streams as ``hipStream_t`` handles (by default
torch's current stream).  A non-OK status raises :class:`HTError`.

The library must be built in-tree (``python -m block_planner_amd.build`` or
``__graft_entry__.build()``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libht.so")
# The same library built with the fused MLP's phase timestamps
# (block_planner_amd.build, -DHT_MLP_PHASES); it also exports ht_mlp_phases.
PHASES_LIB_PATH = os.path.join(HERE, "libht_phases.so")

HT_INT4, HT_INT8, HT_BF16, HT_FP16, HT_FP32 = range(5)
HT_ACT_NONE, HT_ACT_RELU = 0, 1
HT_PATH_AUTO, HT_PATH_GEMV, HT_PATH_FUSED, HT_PATH_GEMM, HT_PATH_GEMV_MFMA, HT_PATH_GEMM_I8, HT_PATH_W8A8 = 0, 1, 2, 3, 4, 5, 6
HT_LAYOUT_VERSION = 1
STATUS = {0: "HT_OK", 1: "HT_EINVAL", 2: "HT_ESHAPE", 3: "HT_EALIGN", 4: "HT_ESMALL", 5: "HT_EHIP"}

# Every symbol include/ht.h declares.
EXPORTS = ("ht_status_string", "ht_plan_params_default", "ht_plan", "ht_plan_counts",
           "ht_pack_bytes", "ht_pack", "ht_refresh_bytes", "ht_refresh", "ht_refresh_desc", "ht_check_packed",
           "ht_linear_workspace", "ht_linear_forward",
           "ht_linear_forward_noalloc",
           "ht_linear_backward_workspace", "ht_linear_backward_data", "ht_linear_backward_weight",
           "ht_mlp_workspace", "ht_workspace_init", "ht_mlp_forward")


class HTError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({ht_status_string(code)})")


class PlanParams(ctypes.Structure):
    _fields_ = [("eps_int4", ctypes.c_double), ("eps_int8", ctypes.c_double),
                ("eps_bf16", ctypes.c_double), ("eps_fp16", ctypes.c_double),
                ("prefer_bf16", ctypes.c_int32), ("force_format", ctypes.c_int32)]


class PackedWeight(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("row_tile", ctypes.c_int64),
                ("n_tiles", ctypes.c_int64), ("counts", ctypes.c_int64 * 5),
                ("off_kbidx", ctypes.c_uint64), ("off_ids", ctypes.c_uint64 * 5),
                ("off_scale", ctypes.c_uint64 * 2), ("off_payload", ctypes.c_uint64 * 5),
                ("bytes", ctypes.c_uint64), ("layout_version", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("base", ctypes.c_void_p)]


_lib = None


def use_library(path: str) -> None:
    """Load the library from `path` instead (e.g. PHASES_LIB_PATH); must be
    called before the first load."""
    global LIB_PATH
    if _lib is not None and os.path.abspath(path) != os.path.abspath(LIB_PATH):
        raise RuntimeError("the library is already loaded")
    LIB_PATH = path


def load() -> ctypes.CDLL:
    """Load the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m block_planner_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    St = ctypes.c_int
    lib.ht_status_string.restype = ctypes.c_char_p
    lib.ht_status_string.argtypes = [St]
    lib.ht_plan_params_default.restype = None
    lib.ht_plan_params_default.argtypes = [ctypes.POINTER(PlanParams)]
    lib.ht_plan.restype = St
    lib.ht_plan.argtypes = [P, I64, I64, I64, ctypes.POINTER(PlanParams), P, P]
    lib.ht_plan_counts.restype = St
    lib.ht_plan_counts.argtypes = [P, I64, I64, P, P]
    lib.ht_pack_bytes.restype = St
    lib.ht_pack_bytes.argtypes = [I64, I64, I64, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_size_t)]
    lib.ht_pack.restype = St
    lib.ht_pack.argtypes = [P, I64, I64, I64, P, I64, ctypes.POINTER(ctypes.c_int64), P, ctypes.c_size_t,
                            ctypes.POINTER(PackedWeight), P]
    lib.ht_refresh_bytes.restype = St
    lib.ht_refresh_bytes.argtypes = [I64, I64, I64, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    lib.ht_refresh.restype = St
    lib.ht_refresh.argtypes = [P, I64, I64, I64, ctypes.POINTER(PlanParams), I64, P, P, ctypes.c_size_t, P, P,
                               ctypes.c_size_t, P]
    lib.ht_refresh_desc.restype = St
    lib.ht_refresh_desc.argtypes = [I64, I64, I64, ctypes.POINTER(ctypes.c_int64), P, ctypes.c_size_t,
                                    ctypes.POINTER(PackedWeight)]
    lib.ht_check_packed.restype = St
    lib.ht_check_packed.argtypes = [ctypes.POINTER(PackedWeight), P, ctypes.c_size_t, P]
    lib.ht_linear_workspace.restype = St
    lib.ht_linear_workspace.argtypes = [ctypes.POINTER(PackedWeight), I64, I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.ht_linear_forward.restype = St
    lib.ht_linear_forward.argtypes = [ctypes.POINTER(PackedWeight), P, I64, I64, P, I64, I32, I32, P,
                                      ctypes.c_size_t, P]
    lib.ht_linear_forward_noalloc.restype = St
    lib.ht_linear_forward_noalloc.argtypes = [ctypes.POINTER(PackedWeight), P, I64, I64, P, I64, I32, I32, P]
    lib.ht_linear_backward_workspace.restype = St
    lib.ht_linear_backward_workspace.argtypes = [ctypes.POINTER(PackedWeight), I64, ctypes.POINTER(ctypes.c_size_t)]
    lib.ht_linear_backward_data.restype = St
    lib.ht_linear_backward_data.argtypes = [ctypes.POINTER(PackedWeight), P, I64, I64, P, I64, P, ctypes.c_size_t, P]
    lib.ht_linear_backward_weight.restype = St
    lib.ht_linear_backward_weight.argtypes = [P, I64, I64, P, I64, I64, I64, P, I64, I32, P]
    lib.ht_mlp_workspace.restype = St
    lib.ht_mlp_workspace.argtypes = [ctypes.POINTER(ctypes.POINTER(PackedWeight)), I32, I64,
                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.ht_workspace_init.restype = St
    lib.ht_workspace_init.argtypes = [P, ctypes.c_size_t, P]
    lib.ht_mlp_forward.restype = St
    lib.ht_mlp_forward.argtypes = [ctypes.POINTER(ctypes.POINTER(PackedWeight)), I32, P, I64, I64, P, I64, P, I32,
                                   P, ctypes.c_size_t, P]
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise HTError(fn, code)


def ht_status_string(code: int) -> str:
    return load().ht_status_string(code).decode()


def ht_plan_params_default() -> PlanParams:
    p = PlanParams()
    load().ht_plan_params_default(ctypes.byref(p))
    return p


def ht_plan(W, fmt_map, params: PlanParams | None = None, stream=None, N=None, K=None, ldw=None) -> None:
    """W: fp32 [N, K] (row stride ldw); fmt_map: uint8 [N, K/64]."""
    N = W.shape[0] if N is None else N
    K = W.shape[1] if K is None else K
    ldw = W.stride(0) if ldw is None else ldw
    pp = ctypes.byref(params) if params is not None else None
    _check("ht_plan", load().ht_plan(_ptr(W), N, K, ldw, pp, _ptr(fmt_map), _stream(stream)))


def ht_plan_counts(fmt_map, counts5, N=None, K=None, stream=None) -> None:
    N = fmt_map.shape[0] if N is None else N
    K = fmt_map.shape[1] * 64 if K is None else K
    _check("ht_plan_counts", load().ht_plan_counts(_ptr(fmt_map), N, K, _ptr(counts5), _stream(stream)))


def ht_pack_bytes(N: int, K: int, row_tile: int, counts) -> int:
    c = (ctypes.c_int64 * 5)(*[int(v) for v in counts])
    out = ctypes.c_size_t(0)
    _check("ht_pack_bytes", load().ht_pack_bytes(N, K, row_tile, c, ctypes.byref(out)))
    return out.value


def ht_pack(W, fmt_map, row_tile: int, counts, buf, stream=None, N=None, K=None, ldw=None,
            buf_bytes=None) -> PackedWeight:
    N = W.shape[0] if N is None else N
    K = W.shape[1] if K is None else K
    ldw = W.stride(0) if ldw is None else ldw
    c = (ctypes.c_int64 * 5)(*[int(v) for v in counts])
    desc = PackedWeight()
    nbytes = buf.numel() * buf.element_size() if buf_bytes is None else buf_bytes
    _check("ht_pack", load().ht_pack(_ptr(W), N, K, ldw, _ptr(fmt_map), row_tile, c, _ptr(buf), nbytes,
                                     ctypes.byref(desc), _stream(stream)))
    return desc


def ht_refresh_bytes(N: int, K: int, row_tile: int) -> tuple:
    """(buf_bytes, ws_bytes) for ht_refresh."""
    b, w = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("ht_refresh_bytes", load().ht_refresh_bytes(N, K, row_tile, ctypes.byref(b), ctypes.byref(w)))
    return b.value, w.value


def ht_refresh(W, fmt_map, buf, counts5, ws, params: PlanParams | None = None, row_tile: int = 16, stream=None,
               N=None, K=None, ldw=None, buf_bytes=None, ws_bytes=None) -> None:
    N = W.shape[0] if N is None else N
    K = W.shape[1] if K is None else K
    ldw = W.stride(0) if ldw is None else ldw
    bb = buf.numel() * buf.element_size() if buf_bytes is None else buf_bytes
    wb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    pp = ctypes.byref(params) if params is not None else None
    _check("ht_refresh", load().ht_refresh(_ptr(W), N, K, ldw, pp, row_tile, _ptr(fmt_map), _ptr(buf), bb,
                                           _ptr(counts5), _ptr(ws), wb, _stream(stream)))


def ht_refresh_desc(N: int, K: int, row_tile: int, counts, buf, buf_bytes=None) -> PackedWeight:
    c = (ctypes.c_int64 * 5)(*[int(v) for v in counts])
    bb = buf.numel() * buf.element_size() if buf_bytes is None else buf_bytes
    desc = PackedWeight()
    _check("ht_refresh_desc", load().ht_refresh_desc(N, K, row_tile, c, _ptr(buf), bb, ctypes.byref(desc)))
    return desc


def ht_check_packed(desc: PackedWeight, host_buf, fmt_out=None) -> None:
    """host_buf, fmt_out: numpy arrays in host memory (uint8 bytes of the
    packed buffer; uint8 [N, K/64] receiving the map the index describes)."""
    fp = None if fmt_out is None else fmt_out.ctypes.data
    _check("ht_check_packed", load().ht_check_packed(ctypes.byref(desc), host_buf.ctypes.data, host_buf.nbytes, fp))


def ht_linear_workspace(desc: PackedWeight, M: int, path: int = HT_PATH_AUTO) -> int:
    out = ctypes.c_size_t(0)
    _check("ht_linear_workspace", load().ht_linear_workspace(ctypes.byref(desc), M, path, ctypes.byref(out)))
    return out.value


def ht_linear_forward(desc: PackedWeight, x, y, act: int = HT_ACT_NONE, path: int = HT_PATH_AUTO, ws=None,
                      stream=None, M=None, ldx=None, ldy=None, ws_bytes=None) -> None:
    M = x.shape[0] if M is None else M
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    wsb = (ws.numel() * ws.element_size() if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check("ht_linear_forward", load().ht_linear_forward(ctypes.byref(desc), _ptr(x), M, ldx, _ptr(y), ldy, act,
                                                         path, _ptr(ws), wsb, _stream(stream)))


def ht_linear_forward_noalloc(desc: PackedWeight, x, y, act: int = HT_ACT_NONE, path: int = HT_PATH_AUTO,
                              stream=None, M=None, ldx=None, ldy=None) -> None:
    M = x.shape[0] if M is None else M
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    _check("ht_linear_forward_noalloc", load().ht_linear_forward_noalloc(ctypes.byref(desc), _ptr(x), M, ldx, _ptr(y),
                                                                         ldy, act, path, _stream(stream)))


def ht_linear_backward_workspace(desc: PackedWeight, M: int) -> int:
    out = ctypes.c_size_t(0)
    _check("ht_linear_backward_workspace", load().ht_linear_backward_workspace(ctypes.byref(desc), M,
                                                                               ctypes.byref(out)))
    return out.value


def ht_linear_backward_data(desc: PackedWeight, dy, dx, ws=None, stream=None, M=None, lddy=None, lddx=None,
                            ws_bytes=None) -> None:
    M = dy.shape[0] if M is None else M
    lddy = dy.stride(0) if lddy is None else lddy
    lddx = dx.stride(0) if lddx is None else lddx
    wsb = (ws.numel() * ws.element_size() if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check("ht_linear_backward_data", load().ht_linear_backward_data(ctypes.byref(desc), _ptr(dy), M, lddy, _ptr(dx),
                                                                     lddx, _ptr(ws), wsb, _stream(stream)))


def ht_linear_backward_weight(dy, x, dw, accumulate=False, stream=None, M=None, N=None, K=None, lddy=None,
                              ldx=None, lddw=None) -> None:
    """x: bf16 (or its uint16 bits) [M, K]; dy fp32 [M, N]; dw fp32 [N, K]."""
    M = dy.shape[0] if M is None else M
    N = dw.shape[0] if N is None else N
    K = dw.shape[1] if K is None else K
    lddy = dy.stride(0) if lddy is None else lddy
    ldx = x.stride(0) if ldx is None else ldx
    lddw = dw.stride(0) if lddw is None else lddw
    _check("ht_linear_backward_weight", load().ht_linear_backward_weight(_ptr(dy), M, lddy, _ptr(x), ldx, N, K,
                                                                         _ptr(dw), lddw, 1 if accumulate else 0,
                                                                         _stream(stream)))


def _desc_array(descs):
    arr = (ctypes.POINTER(PackedWeight) * len(descs))(*[ctypes.pointer(d) for d in descs])
    return arr


def ht_mlp_workspace(descs, M: int) -> int:
    out = ctypes.c_size_t(0)
    _check("ht_mlp_workspace", load().ht_mlp_workspace(_desc_array(descs), len(descs), M, ctypes.byref(out)))
    return out.value


def ht_workspace_init(ws, stream=None, ws_bytes=None) -> None:
    wsb = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check("ht_workspace_init", load().ht_workspace_init(_ptr(ws), wsb, _stream(stream)))


def ht_mlp_forward(descs, x, y, act_dump=None, path: int = HT_PATH_AUTO, ws=None, stream=None, M=None, ldx=None,
                   ldy=None, ws_bytes=None, desc_array=None) -> None:
    M = x.shape[0] if M is None else M
    ldx = x.stride(0) if ldx is None else ldx
    ldy = y.stride(0) if ldy is None else ldy
    wsb = (ws.numel() * ws.element_size() if ws is not None else 0) if ws_bytes is None else ws_bytes
    arr = _desc_array(descs) if desc_array is None else desc_array
    _check("ht_mlp_forward", load().ht_mlp_forward(arr, len(descs), _ptr(x), M, ldx, _ptr(y), ldy,
                                                   _ptr(act_dump), path, _ptr(ws), wsb, _stream(stream)))
