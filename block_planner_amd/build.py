"""Build the gfx950 library ``block_planner_amd/libht.so`` with hipcc.

Always recompiles (the caller asked for a build).  Each source is compiled to
an object in ``_build/`` in parallel, then linked into the in-tree shared
library that the Python binding loads.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libht.so")
# The fused MLP's phase-timestamp variant (compiled with -DHT_MLP_PHASES),
# used only by bench.py --only phases.
OUT_PHASES = os.path.join(HERE, "libht_phases.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "plan.hip", "pack.hip", "linear.hip", "gemm.hip", "gemm_xw.hip", "gemm_i8.hip", "gemv_mfma.hip", "mlp.hip", "backward.hip", "bwd_gemm.hip", "noalloc.hip", "refresh.hip"]

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 are generated.
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def _compile(src: str, tag: str = "", defines=()) -> str:
    obj = os.path.join(BUILD_DIR, tag + os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, phases: bool = True) -> str:
    """Build libht.so; with `phases` also libht_phases.so (the same sources
    with the fused MLP's phase timestamps compiled in)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
        pobj = ex.submit(_compile, "mlp.hip", "phases_", ("-DHT_MLP_PHASES",)) if phases else None
        pobj = pobj.result() if pobj else None
    _link(objs, OUT)
    if verbose:
        print("built", OUT)
    if pobj:
        _link([pobj if o.endswith("/mlp.hip.o") else o for o in objs], OUT_PHASES)
        if verbose:
            print("built", OUT_PHASES)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
