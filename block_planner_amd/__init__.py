"""MI355X (gfx950) per-block mixed-precision quantized linear.

The compute path lives in the in-tree HIP library ``libht.so`` (C ABI in
``include/ht.h``); ``binding`` forwards to it and ``api`` allocates buffers
with torch around those calls.  Importing this package loads nothing: the
library is loaded on first use and a missing build raises.
"""
__all__ = ["binding", "api", "workloads"]
