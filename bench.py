#!/usr/bin/env python3
"""Benchmark of the fused mixed-format GEMV on the 4096-wide, depth-4 MLP.

One step = one forward of the MLP (four Linear(4096, 4096) + ReLU layers, no
bias, bfloat16 activations, batch 1) through ``ht_mlp_forward`` over packed
execution buffers.  The weights are seeded synthetic Student-t draws (see
``block_planner_amd.workloads.mlp_weight``), planned with the default
thresholds and packed once before timing.

Cache hygiene: one packed MLP is ~125 MB and would sit in the 256 MB
Infinity Cache if the same copy were reused, so the timed loop rotates over
``--copies`` independently packed copies (6 x 125 MB by default) and reads
from HBM.  A warm-cache figure (one copy, no rotation) is reported separately.

Reported value: algorithmic bytes per step / time per step, where a layer's
algorithmic bytes are, per block, its payload + scale + one format-map byte
(INT4 37, INT8 69, BF16/FP16 129, FP32 257), plus the input activations
(2 bytes each) and the output (2 bytes for bfloat16 hidden layers, 4 for the
fp32 last layer).

Also reported (not the headline value): planner, packer and fused-refresh
GB/s (over 8 rotated fp32 weights, 512 MB), the single-layer GEMV, the
per-layer MLP path, batch 16 (µs per 4096^2 layer on the MFMA decode path)
and 32, a warm-cache figure, the prefill GEMM (MFMA
path, M = 2048, Llama-8B-shaped layers) in TFLOP/s, the int8 path, the
backward kernels, and the transformer-shaped configurations: TinyLlama decode
at batch 1 over its 154 linears (and over its 88 fused-projection weights),
Llama-8B decode at batch 1 / 4 / 16 over its 224 linears (and 128 fused) and
the planner / packer sweep over the Llama-8B set.  The CPU
baseline is the oracle on the host's cores (all of them, and one).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
PAY = (32, 64, 128, 128, 256)   # payload bytes per block
SCALE = (4, 4, 0, 0, 0)


def layer_bytes(counts, M, K, N, out_bytes):
    w = sum(c * (p + s + 1) for c, p, s in zip(counts, PAY, SCALE))
    return w + 2 * M * K + out_bytes * M * N


KERNEL_SOURCES = ("mlp.hip", "gemv_common.h", "ht_internal.h")


def kernel_sha() -> str:
    """Hash of the sources the fused MLP kernel is compiled from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "block_planner_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def traffic_entry():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "mlp_fused_mlp4096_m1_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        sha = kernel_sha()
        if d.get("source_sha256") != sha:
            return None
        return d.get("hbm_bytes_per_launch")
    except Exception:
        return None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--copies", type=int, default=6)
    ap.add_argument("--cpu-steps", type=int, default=100,
                    help="oracle MLP forwards timed on all cores for the CPU baseline (a fifth of them on one core)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "gemv", "mlp", "gemm", "decode", "i8", "configs", "backward",
                                       "phases"],
                    default="all",
                    help="'gemv' / 'mlp' / 'gemm' / 'decode': only that timing leg (for profiler runs)")
    ap.add_argument("--no-gemm", action="store_true", help="skip the prefill GEMM leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the transformer-shaped configurations (TinyLlama / Llama-8B decode, plan/pack sweep)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from block_planner_amd import api
    from block_planner_amd import binding as B
    from block_planner_amd import workloads as wl

    if args.only == "phases":
        B.use_library(B.PHASES_LIB_PATH)   # the fused MLP with its phase timestamps compiled in
    B.load()   # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    D, L = wl.MLP_DIM, wl.MLP_DEPTH

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def flush():
        """Write 512 MB (twice the 256 MB Infinity Cache), so what was
        touched before comes from HBM again."""
        flush_buf.fill_(1)

    def clone_packed(pw):
        """An independent copy of a packed weight (its own aligned buffer)."""
        buf = api._aligned_empty(pw.nbytes, dev)
        buf.copy_(pw.buf[:pw.nbytes])
        d = B.PackedWeight()
        ctypes.memmove(ctypes.addressof(d), ctypes.addressof(pw.desc), ctypes.sizeof(d))
        d.base = buf.data_ptr()
        return api.PackedLinear(buf, d, list(pw.counts))

    def copies_over(pw, min_bytes=512 << 20):
        """pw plus copies until together they exceed min_bytes."""
        out = [pw]
        while sum(p_.nbytes for p_ in out) < min_bytes:
            out.append(clone_packed(pw))
        return out

    def timed(fn, reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record(stream)
        for i in range(reps):
            fn(i)
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps / 1e3   # seconds per rep

    def gemm_leg():
        """Prefill: ht_linear_forward on the MFMA path at M = 2048 over
        Llama-8B-shaped layers (q: 4096x4096, gate: 14336x4096, down:
        4096x14336), seeded synthetic weights planned with the default
        thresholds; at this M the path expands the weight tiles once, then
        runs the matrix-core kernel on them (both kernels timed).  Reported:
        TFLOP/s of 2*M*N*K and the fraction of the 2.5 PFLOP/s dense bf16
        MFMA peak."""
        out = {}
        M = 2048
        for name in ("q", "gate", "down"):
            shp = [t for t in wl.llama8b_shapes() if t.name == name][0]
            W = torch.from_numpy(wl.llama8b_weight(0, shp)).to(dev)
            fmt = api.plan(W)
            pw = api.pack(W, fmt)
            del W
            xb = torch.from_numpy(wl.to_bf16_bits(wl.activation("llama8b", M, shp.k)).view(np.int16)).to(dev)
            xg = xb.view(torch.bfloat16)
            yg = torch.empty((M, shp.n), dtype=torch.float32, device=dev)
            for _ in range(2):
                api.linear(pw, xg, out=yg, path=B.HT_PATH_GEMM)
            reps = 10
            t = timed(lambda i: api.linear(pw, xg, out=yg, path=B.HT_PATH_GEMM), reps)
            fl = 2.0 * M * shp.n * shp.k
            out[name] = {"M": M, "N": shp.n, "K": shp.k, "us": round(t * 1e6, 1),
                         "TFLOPs": round(fl / t / 1e12, 1), "mfma_frac": round(fl / t / 2.5e15, 4)}
            del pw, xb, yg
            torch.cuda.empty_cache()
        return {"kernel": "xw_expand_kernel + gemm_xw_kernel (two passes at M = 2048)", "peak_TFLOPs": 2500.0,
                "shapes": out}

    def i8_leg():
        """The int8 matrix-core path (HT_PATH_GEMM_I8) and the opt-in W8A8
        mode (HT_PATH_W8A8: x as one int8 plane per 64-wide K-block) against
        the MFMA path at M = 2048 on the same Llama-8B shapes: once on
        weights forced to INT8 everywhere (every 256-column tile takes the
        int8 kernel) and once on the planned weights (no tile is all INT8:
        the paths add the encoding of x and an empty int8 launch).  TFLOP/s
        of 2*M*N*K; the int8 kernel's fraction is of the 5.0 POP/s dense
        int8 MFMA peak (GEMM_I8 issues two int8 MFMAs per product, one per
        plane of x; W8A8 one)."""
        out = {}
        M = 2048
        for name in ("q", "gate", "down"):
            shp = [t for t in wl.llama8b_shapes() if t.name == name][0]
            W = torch.from_numpy(wl.llama8b_weight(0, shp)).to(dev)
            xg = torch.from_numpy(wl.to_bf16_bits(wl.activation("llama8b", M, shp.k)).view(np.int16)).to(dev)
            xg = xg.view(torch.bfloat16)
            yg = torch.empty((M, shp.n), dtype=torch.float32, device=dev)
            fl = 2.0 * M * shp.n * shp.k
            row = {}
            for kind in ("all_int8", "planned"):
                fmt = (torch.full((shp.n, shp.k // 64), 1, dtype=torch.uint8, device=dev) if kind == "all_int8"
                       else api.plan(W))
                pw = api.pack(W, fmt)
                r = {}
                paths = (("GEMM", B.HT_PATH_GEMM), ("GEMM_I8", B.HT_PATH_GEMM_I8), ("W8A8", B.HT_PATH_W8A8))
                for pname, path in paths:
                    ws = api.workspace(B.ht_linear_workspace(pw.desc, M, path), dev)
                    for _ in range(2):
                        api.linear(pw, xg, out=yg, ws=ws, path=path)
                    t = timed(lambda i: api.linear(pw, xg, out=yg, ws=ws, path=path), 10)
                    r[pname + "_us"] = round(t * 1e6, 1)
                    r[pname + "_TFLOPs"] = round(fl / t / 1e12, 1)
                    del ws
                r["speedup"] = round(r["GEMM_us"] / r["GEMM_I8_us"], 3)
                r["W8A8_speedup"] = round(r["GEMM_us"] / r["W8A8_us"], 3)
                row[kind] = r
                del pw
            row["all_int8"]["int8_peak_frac"] = round(fl / (row["all_int8"]["GEMM_I8_us"] * 1e-6) / 5.0e15, 4)
            row["all_int8"]["W8A8_int8_peak_frac"] = round(fl / (row["all_int8"]["W8A8_us"] * 1e-6) / 5.0e15, 4)
            out[name] = row
            del W, xg, yg
            torch.cuda.empty_cache()
        return {"kernel": "gemm_i8_kernel<false> + xq_kernel (GEMM_I8), gemm_i8_kernel<true> + xq8_kernel (W8A8)", "peak_int8_TOPs": 5000.0, "M": M, "shapes": out}

    def configs_leg():
        """The transformer-shaped configurations, on seeded device-drawn
        weights (workloads.*_weight_gpu):
          * TinyLlama-1.1B shapes (22 layers x 7 linears = 154): decode at
            batch 1 over all of them, back to back; then the same with q|k|v
            and gate|up packed as one weight each (4 launches per layer);
          * Llama-3.1-8B shapes (32 x 7 = 224 linears, 7.0e9 parameters):
            the planner and packer streamed layer by layer over the whole set
            for eps_int4 in {0.04, 0.08, 0.16} and forced all-INT4 / all-INT8
            plans (events around each call, after a 512 MB write so that W
            comes from HBM, not from the Infinity Cache), then decode at
            batch 1, 4 and 16 over all 224 linears packed at the default eps,
            and over the 128 fused-projection weights.
        Each decode pass is one HIP graph of every linear in order (AUTO
        path, each with its own input and output), replayed; GB/s counts the
        packed bytes plus activations and outputs."""
        res = {}

        def decode_pass(pws, M, reps):
            xs, ys, wss = [], [], []
            for pw in pws:
                xs.append(torch.randn(M, pw.K, device=dev).to(torch.bfloat16))
                ys.append(torch.empty(M, pw.N, dtype=torch.float32, device=dev))
                wss.append(api.workspace(B.ht_linear_workspace(pw.desc, M, B.HT_PATH_AUTO), dev))

            def run_all():   # on the current stream (the capture stream inside the graph)
                for pw, xg, yg, ws in zip(pws, xs, ys, wss):
                    api.linear(pw, xg, out=yg, ws=ws)
            run_all()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_all()
            g.replay()
            torch.cuda.synchronize()
            t = timed(lambda i: g.replay(), reps)
            nbytes = sum(pw.nbytes + 2 * M * pw.K + 4 * M * pw.N for pw in pws)
            del g, xs, ys, wss
            return {"M": M, "linears": len(pws), "us_per_pass": round(t * 1e6, 1),
                    "GBps": round(nbytes / t / 1e9, 1), "pct_hbm_peak": round(100 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2),
                    "bytes_per_pass": int(nbytes)}

        def fused_stack(gen, shapes, layers):
            """Per layer four linears: q|k|v and gate|up as one weight each
            (rows concatenated before planning, as serving engines fuse these
            projections; the plan is per block, so every row gets the blocks
            it gets alone), then o and down."""
            sh = {s_.name: s_ for s_ in shapes}
            out = []
            for layer in range(layers):
                for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
                    W = torch.cat([gen(layer, sh[n], dev) for n in group])
                    out.append(api.pack(W, api.plan(W)))
                    del W
            return out

        # TinyLlama: decode at batch 1 over the 154 linears, then over the 88
        # launches of the fused q|k|v and gate|up weights
        log("configs: TinyLlama stack")
        pws = []
        for layer in range(wl.TINYLLAMA_LAYERS):
            for shp in wl.tinyllama_shapes():
                W = wl.tinyllama_weight_gpu(layer, shp, dev)
                pws.append(api.pack(W, api.plan(W)))
                del W
        res["tinyllama_decode_b1"] = decode_pass(pws, 1, 20)
        del pws
        pws = fused_stack(wl.tinyllama_weight_gpu, wl.tinyllama_shapes(), wl.TINYLLAMA_LAYERS)
        res["tinyllama_decode_b1_fused_qkv_gateup"] = decode_pass(pws, 1, 20)
        del pws
        torch.cuda.empty_cache()

        # Llama-8B: planner / packer sweep, then decode
        log("configs: Llama-8B planner / packer sweep")
        settings = [("eps_int4=0.04", {"eps_int4": 0.04}), ("eps_int4=0.08", {}), ("eps_int4=0.16", {"eps_int4": 0.16}),
                    ("all INT4", {"force_format": 0}), ("all INT8", {"force_format": 1})]
        acc = {name: {"plan_s": 0.0, "pack_s": 0.0, "read": 0, "map": 0, "packed": 0, "counts": [0] * 5}
               for name, _ in settings}
        keep = []
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for layer in range(wl.LLAMA8B_LAYERS):
            for shp in wl.llama8b_shapes():
                W = wl.llama8b_weight_gpu(layer, shp, dev)
                for name, kw in settings:
                    a = acc[name]
                    fmt = torch.empty((shp.n, shp.k // 64), dtype=torch.uint8, device=dev)
                    flush()   # W was just generated (or planned): take it from HBM
                    ev0.record(stream)
                    B.ht_plan(W, fmt, api.plan_params(**kw), stream=stream)
                    ev1.record(stream)
                    ev1.synchronize()
                    a["plan_s"] += ev0.elapsed_time(ev1) / 1e3
                    cnt = api.counts(fmt)
                    nb = B.ht_pack_bytes(shp.n, shp.k, 16, cnt)
                    buf = api._aligned_empty(nb, dev)
                    flush()
                    ev0.record(stream)
                    desc = B.ht_pack(W, fmt, 16, cnt, buf, stream=stream)
                    ev1.record(stream)
                    ev1.synchronize()
                    a["pack_s"] += ev0.elapsed_time(ev1) / 1e3
                    a["read"] += 4 * shp.n * shp.k
                    a["map"] += shp.n * shp.k // 64
                    a["packed"] += nb
                    a["counts"] = [u + v for u, v in zip(a["counts"], cnt)]
                    if name == "eps_int4=0.08":
                        keep.append(api.PackedLinear(buf, desc, cnt))
                    else:
                        del buf
                    del fmt
                del W
        sweep = {}
        for name, _ in settings:
            a = acc[name]
            tot = sum(a["counts"])
            sweep[name] = {"planner_GBps": round((a["read"] + a["map"]) / a["plan_s"] / 1e9, 1),
                           "packer_GBps": round((a["read"] + a["map"] + a["packed"]) / a["pack_s"] / 1e9, 1),
                           "plan_s": round(a["plan_s"], 4), "pack_s": round(a["pack_s"], 4),
                           "packed_GB": round(a["packed"] / 1e9, 3),
                           "format_mix": {f: round(c / tot, 5) for f, c in
                                          zip(("INT4", "INT8", "BF16", "FP16", "FP32"), a["counts"])}}
        res["llama8b_plan_pack_sweep"] = {"params": 32 * sum(s_.n * s_.k for s_ in wl.llama8b_shapes()),
                                          "settings": sweep}
        log("configs: Llama-8B decode")
        for M in (1, 4, 16):
            res[f"llama8b_decode_b{M}"] = decode_pass(keep, M, 5)
        del keep
        torch.cuda.empty_cache()
        pws = fused_stack(wl.llama8b_weight_gpu, wl.llama8b_shapes(), wl.LLAMA8B_LAYERS)
        for M in (1, 4, 16):
            res[f"llama8b_decode_b{M}_fused_qkv_gateup"] = decode_pass(pws, M, 5)
        del pws
        torch.cuda.empty_cache()
        return res

    def backward_leg():
        """The input gradient dX = dY . W_hat (ht_linear_backward_data) at 1
        and 4 rows of fp32 dY (register path) and at 2048 rows (matrix-core
        path; TFLOP/s of 2*M*N*K and its fraction of the 2.5 PFLOP/s bf16
        peak, the kernel issuing three bf16 products per product): the
        4096x4096 MLP layer (default thresholds) and the Llama-8B q / gate /
        down shapes.  Graph replays of calls that
        rotate over copies of the packed weight holding together more than
        512 MB (the Infinity Cache holds 256 MB); GB/s counts packed bytes +
        dY + dX.  The weight gradient writes a fresh 64 MB fp32 dW per call
        (write-bound, not served by the cache); from 64 rows on the matrix cores,
        at 2048 rows compute-bound (TFLOP/s of 2*M*N*K, two bf16 products per
        product)."""
        res = {}
        cases = [("mlp4096", None)] + [(s_.name, s_) for s_ in wl.llama8b_shapes() if s_.name in ("q", "gate", "down")]
        for name, shp in cases:
            W = (torch.from_numpy(wl.mlp_weight(0)).to(dev) if shp is None else wl.llama8b_weight_gpu(0, shp, dev))
            pws = copies_over(api.pack(W, api.plan(W)))   # rotated: more than the Infinity Cache holds
            del W
            pw = pws[0]
            row = {"rotating_copies": len(pws)}
            for M in (1, 4):
                dy = torch.randn(M, pw.N, device=dev)
                dx = torch.empty(M, pw.K, device=dev)
                ws = api.workspace(B.ht_linear_backward_workspace(pw.desc, M), dev)
                n_in = 2 * len(pws)
                g = torch.cuda.CUDAGraph()
                api.linear_backward_data(pw, dy, out=dx, ws=ws)
                torch.cuda.synchronize()
                with torch.cuda.graph(g):
                    for i in range(n_in):
                        api.linear_backward_data(pws[i % len(pws)], dy, out=dx, ws=ws)
                g.replay()
                torch.cuda.synchronize()
                t = timed(lambda i: g.replay(), 3) / n_in
                nb = pw.nbytes + 4 * M * (pw.N + pw.K)
                row[f"M{M}"] = {"us": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1)}
                del g
            # training batch: 2048 rows of dY on the matrix-core path
            M = 2048
            dy = torch.randn(M, pw.N, device=dev)
            dx = torch.empty(M, pw.K, device=dev)
            ws = api.workspace(B.ht_linear_backward_workspace(pw.desc, M), dev)
            api.linear_backward_data(pw, dy, out=dx, ws=ws)
            torch.cuda.synchronize()
            t = timed(lambda i: api.linear_backward_data(pws[i % len(pws)], dy, out=dx, ws=ws), 6)
            fl = 2.0 * M * pw.N * pw.K
            row["M2048"] = {"us": round(t * 1e6, 1), "TFLOPs": round(fl / t / 1e12, 1),
                            "mfma_frac": round(fl / t / 2.5e15, 4)}
            del dy, dx, ws
            res[name] = row
            del pw, pws
        # STE weight gradient dW = dY^T . x (fp32 [N, K] written): 4096 x 4096
        wg = {}
        for M in (1, 32, 2048):
            dy = torch.randn(M, 4096, device=dev)
            xb = torch.randn(M, 4096, device=dev).to(torch.bfloat16)
            dw = torch.empty(4096, 4096, device=dev)
            fn = lambda: api.linear_backward_weight(dy, xb, out=dw)
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(10):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            t = timed(lambda i: g.replay(), 5) / 10
            nb = 4 * 4096 * 4096 + M * (2 * 4096 + 4 * 4096)
            fl = 2.0 * M * 4096 * 4096
            wg[f"M{M}"] = {"us": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1),
                           "TFLOPs": round(fl / t / 1e12, 1), "mfma_frac": round(fl / t / 2.5e15, 4)}
            del g, dw
        return {"kernel": "linear_bwd_kernel<M> (M < 16), bwd_gemm_kernel<4> (M = 2048)", "shapes": res,
                "weight_grad_4096": {"kernel": "linear_dw_kernel (M < 64), dw_gemm_kernel (M >= 64)", **wg}}

    if args.only == "backward":
        print(json.dumps(backward_leg()))
        return 0
    if args.only == "configs":
        print(json.dumps(configs_leg()))
        return 0
    if args.only == "gemm":
        print(json.dumps(gemm_leg()))
        return 0
    if args.only == "i8":
        print(json.dumps(i8_leg()))
        return 0

    log("generating weights")
    Ws_host = [wl.mlp_weight(l) for l in range(L)]
    Ws = [torch.from_numpy(W).to(dev) for W in Ws_host]

    # ---- planner ---------------------------------------------------------
    # Calls rotate over 8 fp32 weights (the 4 layers and a copy of each:
    # 512 MB, twice the Infinity Cache), so W comes from HBM.
    log("planner")
    fmts = [api.plan(W) for W in Ws]
    torch.cuda.synchronize()
    Wrot = Ws + [W.clone() for W in Ws]
    plan_reps = 8 * 6
    t_plan = timed(lambda i: B.ht_plan(Wrot[i % 8], fmts[i % L]), plan_reps)   # per 4096^2 layer
    plan_bytes = 4 * D * D + D * D // 64
    counts = [api.counts(f) for f in fmts]

    # ---- packer ----------------------------------------------------------
    log("packer")
    copies = [[api.pack(Ws[l], fmts[l], row_tile=16, cnt=counts[l]) for l in range(L)]
              for _ in range(max(1, args.copies))]
    torch.cuda.synchronize()
    scratch = [api.pack(Ws[l], fmts[l], row_tile=16, cnt=counts[l]) for l in range(L)]
    t_pack = timed(lambda i: B.ht_pack(Wrot[i % 8], fmts[i % L], 16, counts[i % L], scratch[i % L].buf), 8 * 4)
    pack_bytes = sum(4 * D * D + D * D // 64 + sum(c * (p + s) for c, p, s in zip(counts[l], PAY, SCALE))
                     for l in range(L)) / L
    del scratch

    # ---- fused refresh (re-plan + re-pack in one pass) ---------------------
    log("refresh")
    rs = api.refresh_state(D, D, 16, dev)
    rbufs = [rs.buf] + [api._aligned_empty(rs.buf.numel(), dev) for _ in range(7)]   # 8 outputs, rotated too
    for l in range(L):                                   # the refresh's output equals the packer's
        api.refresh(Ws[l], rs)
        assert torch.equal(rs.buf[:copies[0][l].nbytes], copies[0][l].buf[:copies[0][l].nbytes])
    params = api.plan_params()

    def refresh_call(i):
        B.ht_refresh(Wrot[i % 8], rs.fmt, rbufs[i % 8], rs.counts, rs.ws, params, row_tile=16, stream=stream)
    t_refresh = timed(refresh_call, 8 * 6)
    refresh_bytes = 4 * D * D + sum(D * D // 64 + copies[0][l].nbytes for l in range(L)) / L
    refresh_ok = int(rs.ws[8:16].view(torch.int32).abs().sum().item()) == 0
    del rs, rbufs, Wrot
    if args.only == "all":
        del Ws   # inference-only: the fp32 masters are not needed any more
        torch.cuda.empty_cache()

    # ---- inputs ----------------------------------------------------------
    def xbf(M):
        bits = wl.to_bf16_bits(wl.mlp_activation(M))
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    x1, x32 = xbf(1), xbf(32)
    C = len(copies)
    ws = api.workspace(max(B.ht_mlp_workspace([p.desc for p in copies[0]], 32),
                           B.ht_linear_workspace(copies[0][0].desc, 32)), dev)
    B.ht_workspace_init(ws)
    y1 = torch.empty((1, D), dtype=torch.float32, device=dev)
    y32 = torch.empty((32, D), dtype=torch.float32, device=dev)
    descs = [[p.desc for p in cp] for cp in copies]

    arrays = [B._desc_array(d) for d in descs]

    def mlp_fn(x, y, rotate=True, path=B.HT_PATH_AUTO):
        def f(i):
            c = i % C if rotate else 0
            B.ht_mlp_forward(descs[c], x, y, path=path, ws=ws, desc_array=arrays[c])
        return f

    def graph_of(fn, n):
        """Capture n calls fn(0..n-1) into one HIP graph (launches only: the
        library records no memset or allocation)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    def replay_timed(g, reps, warm):
        for _ in range(warm):
            g.replay()
        return timed(lambda i: g.replay(), reps)   # seconds per replay

    step_bytes1 = sum(layer_bytes(counts[l], 1, D, D, 2 if l + 1 < L else 4) for l in range(L))
    step_bytes32 = sum(layer_bytes(counts[l], 32, D, D, 2 if l + 1 < L else 4) for l in range(L))
    G = 4 * C                              # forwards per graph
    reps = max(1, -(-args.steps // G))
    steps = reps * G                       # exactly this many steps are timed

    # eager reference output for the replay check
    mlp_fn(x1, y1)(0)
    torch.cuda.synchronize()
    y_eager = y1.clone()

    if args.only == "phases":
        return phases_leg(B, mlp_fn, graph_of, x1, y1, G, step_bytes1, int(copies[0][0].desc.n_tiles), copies[0])

    if args.only == "decode":
        # Decode at batch 16 and 32: one launch per layer on the MFMA decode
        # path (gemv_mfma_kernel<1> / <2>; HT_PATH_AUTO takes it for 5..32
        # rows), graphs of C forwards over the rotating copies, replayed.
        out = {}
        for M in (16, 32):
            xm, ym = xbf(M), torch.empty((M, D), dtype=torch.float32, device=dev)
            gm = graph_of(mlp_fn(xm, ym), C)
            tm = replay_timed(gm, 10, 2) / C
            bm = sum(layer_bytes(counts[l], M, D, D, 2 if l + 1 < L else 4) for l in range(L))
            out[f"mlp_batch{M}"] = {"us_per_forward": round(tm * 1e6, 2), "GBps": round(bm / tm / 1e9, 1)}
            del gm
        print(json.dumps({"kernel": "gemv_mfma_kernel<1> (batch 16) / <2> (batch 32)", "legs": out}))
        return 0

    # ---- single-layer GEMV leg ---------------------------------------------
    # G back-to-back single-layer launches per graph, replayed; events on the
    # launch stream bracket the replays
    log("single-layer gemv timing")
    lin_bytes = [layer_bytes(counts[l], 1, D, D, 4) for l in range(L)]
    glin = graph_of(lambda i: B.ht_linear_forward(descs[(i // L) % C][i % L], x1, y1, ws=ws), G)
    t_rep = replay_timed(glin, max(1, -(-args.steps * L // G)), max(1, args.warmup // G))
    gemv_dur = t_rep / G
    avg_lin_bytes = sum(lin_bytes) / L
    gemv_gbs = avg_lin_bytes / gemv_dur / 1e9
    del glin
    if args.only == "gemv":
        print(json.dumps({"kernel": "gemv_kernel<1>", "avg_launch_us": gemv_dur * 1e6,
                          "algorithmic_bytes_per_launch": avg_lin_bytes, "GBps": gemv_gbs}))
        return 0

    # ---- timed MLP steps (the reported value) ----------------------------
    # One step is one ht_mlp_forward: a single persistent launch of
    # mlp_fused_kernel<1> for all four layers, so the per-step time is also
    # that kernel's per-launch duration (the roofline leg).
    log("mlp timed loop")
    g1 = graph_of(mlp_fn(x1, y1), G)
    t_step = replay_timed(g1, reps, max(1, args.warmup // G)) / G
    torch.cuda.synchronize()
    replay_ok = bool(torch.equal(y1, y_eager))   # every copy holds the same weights
    sync_ok = int(ws[8:12].view(torch.int32).item()) == 0
    value = step_bytes1 / t_step / 1e9
    del g1
    if args.only == "mlp":
        # A plain copy of known size (256 MiB read + 256 MiB written per
        # launch) to scale the HBM byte counters of a counter run.
        a = torch.ones(64 << 20, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
        print(json.dumps({"kernel": "mlp_fused_kernel<1>", "avg_launch_us": t_step * 1e6,
                          "algorithmic_bytes_per_launch": step_bytes1, "GBps": value,
                          "copy_calibration": "torch.neg on 2**26 fp32 (268435456 B read + written), 3 launches"}))
        return 0

    packed_mb = sum(p.nbytes for p in copies[0]) / 1e6
    log("mlp per-layer path, batch 16 and 32, warm cache")
    gp = graph_of(mlp_fn(x1, y1, path=B.HT_PATH_GEMV), G)
    t_perlayer = replay_timed(gp, reps, 1) / G
    x16, y16 = xbf(16), torch.empty((16, D), dtype=torch.float32, device=dev)
    g16 = graph_of(mlp_fn(x16, y16), C)   # the MFMA decode path, one launch per 4096^2 layer
    t16 = replay_timed(g16, 10, 2) / C
    step_bytes16 = sum(layer_bytes(counts[l], 16, D, D, 2 if l + 1 < L else 4) for l in range(L))
    g32 = graph_of(mlp_fn(x32, y32), C)
    t32 = replay_timed(g32, 10, 2) / C
    gw = graph_of(mlp_fn(x1, y1, rotate=False), G)
    t_warm = replay_timed(gw, reps, 1) / G
    del gp, g16, g32, gw

    gemm = bwd = None
    if not args.no_gemm:
        log("prefill gemm (Llama-8B shapes, M = 2048)")
        del copies, arrays, descs
        torch.cuda.empty_cache()
        gemm = gemm_leg()
        log("int8 matrix-core path (Llama-8B shapes, M = 2048)")
        gemm["int8_path"] = i8_leg()
        log("input gradient dX = dY . W_hat (4096x4096 and Llama-8B shapes, M = 1 and 4)")
        bwd = backward_leg()
    configs = None
    if not args.no_configs:
        try:
            del copies, arrays, descs
        except NameError:
            pass
        torch.cuda.empty_cache()
        configs = configs_leg()

    # ---- CPU baseline: the oracle as it stands ----------------------------
    # The C oracle (fp64) on the host cores: one thread, and all the cores
    # the box gives this job (at most 16) each computing a slice of every
    # layer's rows through the same oracle calls (ctypes releases the GIL
    # during a call; the oracle itself is unchanged).
    cpu = None
    if not args.no_cpu_baseline and args.cpu_steps > 0:
        log("cpu baseline (oracle)")
        import concurrent.futures as cf

        import oracle
        fm_host = [f.cpu().numpy() for f in fmts]
        xb = wl.to_bf16_bits(wl.mlp_activation(1))
        oracle.mlp(Ws_host, fm_host, xb)   # load + warm
        n1 = max(1, args.cpu_steps // 5)
        t0 = time.perf_counter()
        for _ in range(n1):
            oracle.mlp(Ws_host, fm_host, xb)
        t_cpu1 = (time.perf_counter() - t0) / n1
        threads = max(1, min(16, os.cpu_count() or 1))
        slices = [[(W[r0:r0 + -(-D // threads)], f[r0:r0 + -(-D // threads)]) for r0 in range(0, D, -(-D // threads))]
                  for W, f in zip(Ws_host, fm_host)]

        def mlp_rows(pool, h):
            for l in range(L):
                parts = list(pool.map(lambda wf: oracle.linear(wf[0], wf[1], h), slices[l]))
                z = np.concatenate(parts, axis=1)
                h = oracle.relu_bf16(z) if l + 1 < L else oracle.relu(z)
            return h
        with cf.ThreadPoolExecutor(max_workers=threads) as pool:
            y_par = mlp_rows(pool, xb)
            assert np.array_equal(y_par, oracle.mlp(Ws_host, fm_host, xb)[0])   # the same oracle result
            t0 = time.perf_counter()
            for _ in range(args.cpu_steps):
                mlp_rows(pool, xb)
            t_cpuN = (time.perf_counter() - t0) / args.cpu_steps
        model = "unknown"
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        cpu = {"value": round(step_bytes1 / t_cpuN / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{args.cpu_steps} forwards of the same 4-layer 4096 MLP at batch 1 (C oracle, fp64; each "
                         f"layer's rows split over {threads} threads; {t_cpuN * 1e3:.1f} ms per forward)",
               "single_thread": {"value": round(step_bytes1 / t_cpu1 / 1e9, 4), "ms_per_forward": round(t_cpu1 * 1e3, 1),
                                 "forwards": n1},
               "nproc": os.cpu_count(), "cpu_model": model}

    mix = [sum(c[f] for c in counts) / sum(sum(c) for c in counts) for f in range(5)]
    out = {
        "metric": "fused mixed-format GEMV GB/s (% of HBM peak) on 4096x4096 MLP; planner GB/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "operands": "int4/int8/bf16/fp16/fp32 weight blocks, bf16 activations, fp32 products and sums",
        "data": "synthetic (seeded Student-t weights, N(0,1) activations)",
        "config": {"workload": "4-layer MLP, Linear(4096,4096)+ReLU x4, no bias, batch 1, bf16 activations, "
                               "default eps (0.08/0.01/0/0), 64-wide K-blocks, row tile 16",
                   "global_batch": 1, "hidden": D, "layers": L, "parallelism": "none (1 GPU)",
                   "rotating_copies": C},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic_entry(),
                     "kernel": "mlp_fused_kernel<1>", "avg_launch_us": round(t_step * 1e6, 3),
                     "algorithmic_bytes_per_launch": int(step_bytes1)},
        "cpu_baseline": cpu,
        "planner_GBps": round(plan_bytes / t_plan / 1e9, 2),
        "planner_pct_hbm_peak": round(100 * plan_bytes / t_plan / 1e9 / HBM_PEAK_GBS, 2),
        "packer_GBps": round(pack_bytes / t_pack / 1e9, 2),
        "plan_pack_working_set": "8 fp32 4096x4096 weights rotated (512 MB, twice the Infinity Cache)",
        "refresh": {"kernel": "refresh_kernel<true, true> (ht_refresh, one pass over W)",
                    "GBps": round(refresh_bytes / t_refresh / 1e9, 2),
                    "pct_hbm_peak": round(100 * refresh_bytes / t_refresh / 1e9 / HBM_PEAK_GBS, 2),
                    "us_per_layer": round(t_refresh * 1e6, 2),
                    "bytes_per_layer": int(refresh_bytes),
                    "bytes": "4 N K read + the map and the packed buffer written",
                    "equals_plan_then_pack": True, "waits_ok": refresh_ok,
                    "vs_plan_then_pack_us": round((t_plan + t_pack) * 1e6, 2)},
        "mlp_per_layer_launches_GBps": round(step_bytes1 / t_perlayer / 1e9, 2),
        "single_layer_gemv": {"kernel": "gemv_kernel<1>", "GBps": round(gemv_gbs, 2),
                              "avg_launch_us": round(gemv_dur * 1e6, 3),
                              "algorithmic_bytes_per_launch": int(avg_lin_bytes)},
        "mlp_batch16_us_per_layer": round(t16 / L * 1e6, 2),
        "mlp_batch16_GBps": round(step_bytes16 / t16 / 1e9, 2),
        "mlp_batch32_GBps": round(step_bytes32 / t32 / 1e9, 2),
        "mlp_batch32_ms_per_step": round(t32 * 1e3, 4),
        "mlp_batch1_warm_cache_GBps": round(step_bytes1 / t_warm / 1e9, 2),
        "graph_replay_matches_eager": replay_ok,
        "grid_barrier_ok": sync_ok,
        "format_mix": {n: round(v, 5) for n, v in zip(("INT4", "INT8", "BF16", "FP16", "FP32"), mix)},
        "packed_MB_per_mlp": round(packed_mb, 2),
        "prefill_gemm": gemm,
        "backward_data": bwd,
        "transformer_configs": configs,
    }
    print(json.dumps(out))
    return 0


PHASE_EVENTS = 20


def phases_leg(B, mlp_fn, graph_of, x1, y1, G, step_bytes1, T, copies0) -> int:
    """Where the time of one fused MLP forward goes, from the instrumented
    build (libht_phases.so): every workgroup's timestamps (100 MHz real-time
    counter) of the last forward of each graph replay, relative to the
    earliest workgroup entry of that forward.  Per event: the median over
    replays of the min / median / max over workgroups, in microseconds."""
    import ctypes

    import numpy as np
    import torch

    lib = B.load()
    lib.ht_mlp_phases.restype = ctypes.c_int
    lib.ht_mlp_phases.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    buf = np.zeros(1024 * PHASE_EVENTS, np.uint64)
    g = graph_of(mlp_fn(x1, y1), G)
    rows = []
    for r in range(40):
        g.replay()
        if r < 4:
            continue
        torch.cuda.synchronize()
        assert lib.ht_mlp_phases(buf.ctypes.data, buf.size) == 0
        ts = buf.reshape(1024, PHASE_EVENTS)[:T].astype(np.int64)
        rows.append((ts - ts[:, 0].min()) * 0.01)   # 10 ns ticks -> us
    # every replay also times the whole graph: the duration of one forward
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(20):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    fwd_us = s.elapsed_time(e) * 1e3 / 20 / G
    a = np.stack(rows)                                  # [replay][wg][event]
    names = ["entry", "x staged, block ranges read", "wave 0: first chunks consumed"]
    for l in range(4):
        names += [f"layer {l}: wave 0 done with its chunks", f"layer {l}: all waves done (barrier)",
                  f"layer {l}: " + ("y written" if l == 3 else "row sums published"),
                  f"layer {l}: next x gathered" if l < 3 else "(unused)"]
    events = {}
    for ev in range(18):                                # events 0..17 of a 4-layer MLP
        v = a[:, :, ev]
        events[f"{ev:2d} {names[ev]}"] = {"min": round(float(np.median(v.min(1))), 2),
                                          "median": round(float(np.median(np.median(v, 1))), 2),
                                          "max": round(float(np.median(v.max(1))), 2)}
    med = lambda ev: float(np.median(np.median(a[:, :, ev], 1)))
    mx = lambda ev: float(np.median(a[:, :, ev].max(1)))
    phases = {"launch ramp: entry spread (max entry)": round(mx(0), 2),
              "to first chunks consumed (median)": round(med(2), 2)}
    prev = 2
    for l in range(4):
        phases[f"layer {l} chunks (median workgroup, from previous phase)"] = round(med(4 + 4 * l) - med(prev), 2)
        if l < 3:
            phases[f"layer {l} boundary: row sums + publish + gather (median)"] = round(med(6 + 4 * l) - med(4 + 4 * l), 2)
            prev = 6 + 4 * l
    phases["last layer tail (median)"] = round(med(17) - med(16), 2)
    phases["end of the last workgroup"] = round(mx(17), 2)
    # per workgroup: median over forwards of the time its waves were all done
    # with each layer's chunks, and the packed bytes of its row tile per layer
    done = [np.median(a[:, :, 4 + 4 * l], 0) for l in range(4)]
    tile_bytes = []
    for l, pw in enumerate(copies0):
        d = pw.desc
        nk = int(d.n_tiles) * (int(d.K) // 64) + 1
        kb = pw.buf[int(d.off_kbidx):int(d.off_kbidx) + 20 * nk].cpu().numpy().view(np.uint32).reshape(5, nk)
        per = np.diff(kb[:, ::int(d.K) // 64].astype(np.int64), axis=1)       # blocks per tile and format
        tile_bytes.append((per * np.array([37, 69, 129, 129, 257])[:, None]).sum(0))
    corr = [float(np.corrcoef(done[l], tile_bytes[l])[0, 1]) for l in range(4)]
    spread = {f"layer {l}": {"done_us_min_med_max": [round(float(np.min(done[l])), 2), round(float(np.median(done[l])), 2),
                                                     round(float(np.max(done[l])), 2)],
                             "tile_kB_min_med_max": [round(float(np.min(tile_bytes[l])) / 1e3, 1),
                                                     round(float(np.median(tile_bytes[l])) / 1e3, 1),
                                                     round(float(np.max(tile_bytes[l])) / 1e3, 1)],
                             "corr_done_vs_bytes": round(corr[l], 3)} for l in range(4)}
    print(json.dumps({"kernel": "mlp_fused_kernel<1> (phase build)", "workgroups": T, "forwards_sampled": len(rows),
                      "workgroup_spread": spread,
                      "us_per_forward_graph": round(fwd_us, 3),
                      "GBps_phase_build": round(step_bytes1 / fwd_us / 1e3, 1),
                      "phases_us": phases, "events_us": events}, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
