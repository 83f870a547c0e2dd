"""GPU parity on the method's edge blocks, through every kernel path.

The edge-block catalogue (workloads.edge_blocks: zero and signed-zero blocks,
fp32-subnormal blocks whose integer scales are subnormal and whose codes
clamp, blocks deep in the subnormal range, huge blocks, integer grids, ties,
bfloat16- and float16-valued blocks, float16 subnormals, the float16
overflow tie, NaN and +-Inf) is laid out in classes of similar magnitude, so
that the bar max|y_gpu - y_oracle| <= 1e-3 * max|y_oracle| of one call is
not decided by a single huge row.  Each class runs under the natural plan
and with every block forced to each format, through HT_PATH_GEMV,
HT_PATH_GEMV_MFMA, HT_PATH_GEMM (single pass, and the two-pass form it
takes from 1024 rows) and HT_PATH_GEMM_I8, through the input gradient, and
through the MLP (single launch and per layer).

Non-finite results.  Positions where the oracle's fp64 result is not finite
must be exactly the GPU's non-finite positions, and NaN where the oracle has
NaN.  The register paths (GEMV, the MLP's single launch, the input gradient)
multiply the decoded values themselves, so +-Inf is kept with its sign.  The
matrix-core paths represent FP16/FP32 entries as a bfloat16 hi plane plus a
lo plane holding bf16(w - hi); an infinite entry makes lo NaN, so where the
oracle has +-Inf those paths give NaN (or the same Inf).  The MLP's ReLU maps
NaN to +0, as the oracle's does.

Left out: the block of 64 entries at 3.4e38.  Its INT4 scale times the
64-term partial overflows fp32 where the fp64 oracle stays finite, and
whether the fp32 sums then give Inf or NaN depends on their order, which the
bar does not define.

A documented bound instead of the bar: fp32-subnormal entries kept as
BF16/FP32 blocks on the matrix-core paths.  bfloat16 keeps only the bits of a
subnormal down to 2^-133, so the hi/lo split can lose up to the whole entry;
the check is |dy| <= bar + sum_k |x_k| |w_hat_k| over those entries.  (On
the register paths the bar holds for them.)

A documented range limit: the int8 path (HT_PATH_GEMM_I8) adds the weight
scale times the exact integer block sums of the encoded x, whose row scale
2^(E-14) multiplies only the finished sum, so its running sums are
2^(14-E) times the output.  Where 2^(14-E_m) sum_k |w_hat[n,k]| |x_hat[m,k]|
reaches FLT_MAX / 2 (weights of magnitude ~1e30 and beyond) that output may
overflow; elsewhere the bar holds, and that is what is checked.
"""
import numpy as np
import pytest
import torch

from block_planner_amd import api
from block_planner_amd import binding as B
from block_planner_amd import workloads as wl

pytestmark = pytest.mark.gpu

INT4, INT8, BF16, FP16, FP32 = 0, 1, 2, 3, 4
TOL = 1e-3

# catalogue rows of workloads.edge_blocks by magnitude class
CLASSES = {
    "unit": [0, 1, 6, 7, 8, 9, 10, 11, 12, 18, 19, 20],
    "subnormal": [0, 1, 2, 3],          # subnormal-scale INT8 blocks, deep-subnormal FP32 blocks
    "fp16small": [0, 13],               # float16 subnormals (fp32-normal)
    "huge": [0, 4],                     # 1e37 entries (x scaled by 1/64)
    "big": [0, 7, 11, 14],              # the float16 overflow tie 65520 among grids
    "nonfinite": [15, 16, 17],          # NaN, +Inf, -Inf, one per chosen row, among unit blocks
}
PLANS = [None, INT4, INT8, BF16, FP16, FP32]
MFMA_PATHS = (B.HT_PATH_GEMV_MFMA, B.HT_PATH_GEMM, B.HT_PATH_GEMM_I8)


def dev():
    return torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_gpu(xbits):
    return gpu(xbits.view(np.int16)).view(torch.bfloat16)


def class_weight(cls, N, K, seed=0):
    """W [N, K]: every block a catalogue row of the class (the first blocks
    run through the whole class).  'nonfinite': one row in four holds one
    non-finite block, the rest are unit blocks, so finite outputs remain."""
    E = wl.edge_blocks(seed)
    rng = np.random.default_rng(seed + 101)
    KB = K // 64
    pool = CLASSES["unit"] if cls == "nonfinite" else CLASSES[cls]
    idx = rng.choice(pool, size=(N, KB))
    idx.reshape(-1)[:len(pool)] = pool
    if cls == "nonfinite":
        bad = CLASSES["nonfinite"]
        for n in range(0, N, 4):
            idx[n, rng.integers(0, KB)] = bad[(n // 4) % len(bad)]
    return np.ascontiguousarray(E[idx].reshape(N, K).astype(np.float32))


def class_x(cls, M, K, seed=0):
    x = wl.activation("edge", M, K, seed=seed)
    if cls == "huge":
        x = x / np.float32(64.0)
    return wl.to_bf16_bits(x)


def plan_for(orc, W, plan):
    return orc.plan(W) if plan is None else orc.plan(W, force=plan)


def check_edge(y, y_or, mfma, what):
    """Failures (a list of strings) of y against y_or under the rules in the
    module docstring."""
    y = np.asarray(y, np.float64)
    out = []
    fin = np.isfinite(y_or)
    if not np.array_equal(np.isfinite(y), fin):
        out.append(f"{what}: non-finite positions differ ({int((np.isfinite(y) != fin).sum())})")
    nan_or = np.isnan(y_or)
    if not np.all(np.isnan(y[nan_or])):
        out.append(f"{what}: not NaN where the oracle is NaN")
    inf_or = np.isinf(y_or)
    ok = y[inf_or] == y_or[inf_or]
    if mfma:
        ok |= np.isnan(y[inf_or])
    if not np.all(ok):
        out.append(f"{what}: infinities differ")
    if fin.any() and np.all(np.isfinite(y[fin])):
        err = float(np.max(np.abs(y[fin] - y_or[fin])))
        ref = float(np.max(np.abs(y_or[fin])))
        if not err <= TOL * ref:
            out.append(f"{what}: max|dy| {err:.3e} > {TOL} * {ref:.3e}")
    return out


def float_subnormal_bound(orc, W, fmt, xbits):
    """sum_k |x_k| |w_hat_k| over entries of BF16/FP16/FP32 blocks whose
    value is a nonzero fp32 subnormal."""
    wh = orc.dequant(W, fmt)
    flt = np.repeat(fmt >= BF16, 64, axis=1)
    sub = flt & (np.abs(wh) < 2.0 ** -126) & (wh != 0)
    xv = np.abs(wl.bf16_bits_to_f32(xbits).astype(np.float64))
    return xv @ np.where(sub, np.abs(wh), 0.0).T


def i8_in_range(orc, W, fmt, xbits):
    """Outputs of the int8 path whose scaled running sums stay below
    FLT_MAX / 2: 2^(14-E_m) sum_k |w_hat[n,k]| |x_hat[m,k]| (bounds every
    partial sum and product in the int8 tiles' accumulation)."""
    hi, lo, sexp = orc.x_planes(xbits)
    xh = np.abs(orc.x_hat(hi, lo, sexp))
    s = np.abs(np.nan_to_num(xh, nan=0.0)) @ np.abs(np.nan_to_num(orc.dequant(W, fmt), nan=0.0, posinf=0.0)).T
    return s * np.ldexp(1.0, -sexp.astype(np.int64))[:, None] < 0.5 * 3.4028234663852886e38


def run(pw, xbits, path, act=B.HT_ACT_NONE):
    y = api.linear(pw, bf16_gpu(xbits), act=act, path=path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


PATH_CASES = [(B.HT_PATH_GEMV, 1), (B.HT_PATH_GEMV, 3), (B.HT_PATH_GEMV_MFMA, 5), (B.HT_PATH_GEMV_MFMA, 32),
              (B.HT_PATH_GEMM, 40), (B.HT_PATH_GEMM, 300), (B.HT_PATH_GEMM_I8, 64)]


@pytest.mark.parametrize("path,M", PATH_CASES)
@pytest.mark.parametrize("cls", list(CLASSES))
def test_edge_linear(orc, cls, path, M):
    """320 x 1024 weights (20 row tiles, K-splits on the split paths) of one
    edge class under the natural plan and every forced format."""
    N, K = 320, 1024
    W = class_weight(cls, N, K)
    x = class_x(cls, M, K, seed=M)
    Wg = gpu(W)
    fails = []
    for plan in PLANS:
        fmt = plan_for(orc, W, plan)
        pw = api.pack(Wg, gpu(fmt))
        what = f"{cls} plan={plan} path={path} M={M}"
        print(what, flush=True)
        y = run(pw, x, path)
        y_or = orc.linear(W, fmt, x)
        if path in MFMA_PATHS and cls == "subnormal" and plan in (BF16, FP32):
            bound = TOL * np.max(np.abs(y_or)) + float_subnormal_bound(orc, W, fmt, x)
            if not np.all(np.abs(y - y_or) <= bound):
                fails.append(f"{what}: beyond the subnormal bound")
            continue
        if path == B.HT_PATH_GEMM_I8:
            keep = i8_in_range(orc, W, fmt, x)
            y, y_or = np.where(keep, y, 0.0), np.where(keep, y_or, 0.0)
        fails += check_edge(y, y_or, path in MFMA_PATHS, what)
    assert not fails, "\n".join(fails)


@pytest.mark.parametrize("cls", list(CLASSES))
def test_edge_linear_two_pass(orc, cls):
    """The MFMA path's two-pass form (weight tiles expanded once, taken from
    1024 rows with at least 192 output tiles): 6144 x 128 weights of one
    edge class at 1024 rows, under the natural plan and every forced format,
    with the MFMA paths' rules."""
    N, K, M = 6144, 128, 1024
    W = class_weight(cls, N, K, seed=7)
    x = class_x(cls, M, K, seed=11)
    Wg = gpu(W)
    fails = []
    for plan in PLANS:
        fmt = plan_for(orc, W, plan)
        pw = api.pack(Wg, gpu(fmt))
        assert B.ht_linear_workspace(pw.desc, M, B.HT_PATH_GEMM) == 48 * 2 * 33 * 1024   # the records
        what = f"{cls} plan={plan} two-pass M={M}"
        print(what, flush=True)
        y = run(pw, x, B.HT_PATH_GEMM)
        y_or = orc.linear(W, fmt, x)
        if cls == "subnormal" and plan in (BF16, FP32):
            bound = TOL * np.max(np.abs(y_or)) + float_subnormal_bound(orc, W, fmt, x)
            if not np.all(np.abs(y - y_or) <= bound):
                fails.append(f"{what}: beyond the subnormal bound")
            continue
        fails += check_edge(y, y_or, True, what)
    assert not fails, "\n".join(fails)


def test_edge_int8_path_range(orc):
    """The int8 path's range limit, from both sides: weights of magnitude
    1e28 (inside it) meet the bar on every output; the catalogue's 1e37
    blocks (outside it: every output's bound exceeds FLT_MAX / 2) are the
    case the limit describes."""
    N, K, M = 320, 1024, 64
    rng = np.random.default_rng(401)
    x = class_x("unit", M, K, seed=5)
    W = (rng.normal(size=(N, K)) * 1e28).astype(np.float32)
    fmt = orc.plan(W, force=INT8)
    assert i8_in_range(orc, W, fmt, x).all()
    pw = api.pack(gpu(W), gpu(fmt))
    assert not check_edge(run(pw, x, B.HT_PATH_GEMM_I8), orc.linear(W, fmt, x), True, "1e28 weights")
    Wh = class_weight("huge", N, K)
    assert i8_in_range(orc, Wh, orc.plan(Wh, force=INT8), class_x("huge", M, K)).mean() < 0.01


@pytest.mark.parametrize("path,M", PATH_CASES)
def test_edge_relu(orc, path, M):
    """The fused ReLU is max(z, 0) of the same fp32 sum with NaN, zero and
    negative values giving +0: bitwise against the call without activation;
    on the register path also the oracle's ReLU."""
    N, K = 320, 1024
    W = class_weight("nonfinite", N, K)
    x = class_x("nonfinite", M, K, seed=M + 7)
    fmt = orc.plan(W)
    pw = api.pack(gpu(W), gpu(fmt))
    z = run(pw, x, path)
    r = run(pw, x, path, act=B.HT_ACT_RELU)
    want = np.where(z > 0, z, np.float32(0.0)).astype(np.float32)
    assert r.tobytes() == want.tobytes()
    assert not np.isnan(r).any() and not np.signbit(r).any()
    if path == B.HT_PATH_GEMV:
        r_or = orc.relu(orc.linear(W, fmt, x))
        assert not check_edge(r, r_or, False, "relu")


@pytest.mark.parametrize("M", [1, 4, 9, 20])
@pytest.mark.parametrize("cls", list(CLASSES))
def test_edge_backward_data(orc, cls, M):
    """dX = dY . W_hat on edge classes, natural plan and every forced format.
    Below 16 rows the register path keeps infinities; from 16 rows the
    matrix-core path splits every weight entry (s * q for integers) into hi
    and lo planes, so an infinity gives NaN and fp32-subnormal entries take
    the documented bound."""
    N, K = 320, 1024
    W = class_weight(cls, N, K)
    rng = np.random.default_rng(300 + M)
    dy = rng.normal(size=(M, N)).astype(np.float32)
    if cls == "huge":
        dy = dy / np.float32(64.0)
    Wg, dyg = gpu(W), gpu(dy)
    fails = []
    for plan in PLANS:
        fmt = plan_for(orc, W, plan)
        pw = api.pack(Wg, gpu(fmt))
        what = f"{cls} plan={plan} M={M}"
        print(what, flush=True)
        dx = api.linear_backward_data(pw, dyg)
        torch.cuda.synchronize()
        dx_or = orc.linear_backward_data(W, fmt, dy)
        if M >= 16 and cls == "subnormal":
            wh = orc.dequant(W, fmt)
            sub = (np.abs(wh) < 2.0 ** -126) & (wh != 0)
            bound = TOL * np.max(np.abs(dx_or)) + np.abs(dy.astype(np.float64)) @ np.where(sub, np.abs(wh), 0.0)
            if not np.all(np.abs(dx.cpu().numpy() - dx_or) <= bound):
                fails.append(f"{what}: beyond the subnormal bound")
            continue
        fails += check_edge(dx.cpu().numpy(), dx_or, M >= 16, what)
    assert not fails, "\n".join(fails)


def _mlp_layers(orc, seed=5):
    """Three layers 256 -> 256 -> 256 -> 128: the first from the non-finite
    class (NaN and +-Inf FP32 blocks among unit blocks), the others unit."""
    Ws = [class_weight("nonfinite", 256, 256, seed), class_weight("unit", 256, 256, seed + 1),
          class_weight("unit", 128, 256, seed + 2)]
    fmts = [orc.plan(W) for W in Ws]
    pws = [api.pack(gpu(W), gpu(f)) for W, f in zip(Ws, fmts)]
    return Ws, fmts, pws


def check_relu_out(hv, r, mfma, half_ulp, what):
    """A ReLU output hv (GPU) against the oracle's r = relu(z): no NaN and no
    -0; +Inf where the oracle has +Inf (on the matrix-core paths also +0,
    the ReLU of the NaN those paths give for an infinity); finite values
    within the bar, plus half a bf16 ulp for a bf16-rounded output."""
    out = []
    if np.isnan(hv).any() or np.signbit(hv).any():
        out.append(f"{what}: NaN or -0 after the ReLU")
    inf_or = np.isinf(r)
    if mfma:
        okinf = (hv[inf_or] == np.inf) | (hv[inf_or] == 0)
        if np.any(np.isinf(hv) & ~inf_or):
            out.append(f"{what}: Inf where the oracle is finite")
    else:
        okinf = hv[inf_or] == np.inf
        if not np.array_equal(np.isinf(hv), inf_or):
            out.append(f"{what}: Inf positions differ")
    if not np.all(okinf):
        out.append(f"{what}: infinities")
    fin = ~inf_or & np.isfinite(hv)
    if fin.any():
        err = np.abs(hv[fin] - r[fin]) - (np.abs(r[fin]) * 2.0 ** -8 if half_ulp else 0.0)
        if not np.max(err) <= TOL * np.max(r[fin]):
            out.append(f"{what}: values beyond the bar")
    return out


@pytest.mark.parametrize("M,path", [(1, B.HT_PATH_FUSED), (3, B.HT_PATH_FUSED), (4, B.HT_PATH_FUSED),
                                    (2, B.HT_PATH_GEMV), (8, B.HT_PATH_AUTO), (40, B.HT_PATH_AUTO)])
def test_edge_mlp(orc, M, path):
    """Teacher-forced per layer: hidden outputs NaN -> +0 and +Inf kept by the
    ReLU, bf16-rounded; the next layer reads the GPU's own activations
    (including infinities).  Rows 8 and 40 run the per-layer matrix-core
    paths (+Inf there may become NaN, then +0 after the ReLU)."""
    Ws, fmts, pws = _mlp_layers(orc)
    x = class_x("unit", M, 256, seed=M + 11)
    ws = api.mlp_workspace(pws, M, dev())
    y, dumps = api.mlp(pws, bf16_gpu(x), dump=True, ws=ws, path=path)
    torch.cuda.synchronize()
    assert int(ws[8:12].view(torch.int32).item()) == 0
    mfma = M >= 4 and path == B.HT_PATH_AUTO
    h_in = x
    fails = []
    for l in range(3):
        r = orc.relu(orc.linear(Ws[l], fmts[l], h_in))
        if l < 2:
            h_gpu = dumps[l].cpu().view(torch.int16).numpy().view(np.uint16)
            fails += check_relu_out(wl.bf16_bits_to_f32(h_gpu).astype(np.float64), r, mfma, True, f"layer {l}")
            h_in = h_gpu
        else:
            fails += check_relu_out(y.cpu().numpy().astype(np.float64), r, mfma, False, "last layer")
    assert not fails, "\n".join(fails)
