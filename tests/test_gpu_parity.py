"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: format maps, codes, scales and packed bytes bit-exact; linear outputs
within max|y_gpu - y_oracle| <= 1e-3 * max|y_oracle| with identical bfloat16
activations on both sides (oracle in fp64).
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


def dev():
    return torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def gpu_plan(W, **kw):
    fmt = api.plan(gpu(W), **kw)
    torch.cuda.synchronize()
    return fmt.cpu().numpy()


def bf16_gpu(xbits):
    return gpu(xbits.view(np.int16)).view(torch.bfloat16)


def check_close(y_gpu, y_or, what=""):
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.max(np.abs(y_gpu - y_or))
    ref = np.max(np.abs(y_or))
    assert np.all(np.isfinite(y_gpu)), what
    assert err <= TOL * ref, f"{what}: max|dy| = {err:.3e} > {TOL} * {ref:.3e}"
    return err / max(ref, 1e-300)


def edge_matrix(rows=32, per_row=4, seed=0):
    E = wl.edge_blocks(seed)
    rng = np.random.default_rng(seed + 5)
    idx = rng.integers(0, E.shape[0], size=(rows, per_row))
    idx[0, :] = np.arange(per_row) % E.shape[0]
    W = E[idx].reshape(rows, per_row * 64)
    return np.ascontiguousarray(W.astype(np.float32))


def finite_rows(W):
    return np.all(np.isfinite(W.reshape(W.shape[0], -1, 64)), axis=-1)


# ---------------------------------------------------------------------------
# Planner
# ---------------------------------------------------------------------------
def test_plan_small_weight(orc):
    W = wl.small_weight()
    np.testing.assert_array_equal(gpu_plan(W), orc.plan(W))


@pytest.mark.parametrize("kw", [
    {}, {"prefer_bf16": False}, {"eps_int4": 0.0, "eps_int8": 0.0},
    {"eps_bf16": 0.004, "eps_fp16": 0.0005}, {"eps_bf16": 0.01, "eps_fp16": 0.01, "prefer_bf16": False},
    {"eps_int4": 0.16}, {"force_format": 0}, {"force_format": 1}, {"force_format": 4},
])
def test_plan_edge_blocks(orc, kw):
    W = edge_matrix()
    oracle_kw = dict(kw)
    force = oracle_kw.pop("force_format", -1)
    np.testing.assert_array_equal(gpu_plan(W, **kw), orc.plan(W, force=force, **oracle_kw))


@pytest.mark.parametrize("shape", [(1, 64), (3, 192), (37, 320), (17, 128), (130, 64 * 88)])
def test_plan_shapes(orc, shape):
    rng = np.random.default_rng(shape[0] * 1000 + shape[1])
    W = (rng.standard_t(3, size=shape) * 0.02).astype(np.float32)
    W.reshape(-1)[rng.choice(W.size, size=max(1, W.size // 200), replace=False)] *= 40
    np.testing.assert_array_equal(gpu_plan(W), orc.plan(W))


def test_plan_near_ties(orc):
    """Thresholds placed at a block's own error ratio and a hair either side
    (the planner screens decisions in fp32 and computes the fp64 trees only
    for blocks too close to call): the map equals the oracle's every time."""
    rng = np.random.default_rng(31)
    W = (rng.standard_t(4, size=(48, 64 * 8)) * 0.02).astype(np.float32)
    err2, nrm2 = orc.block_errors(W)
    for idx in rng.choice(48 * 8, size=12, replace=False):
        n, kb = divmod(int(idx), 8)
        for f, key in ((0, "eps_int4"), (1, "eps_int8")):
            e = float(np.sqrt(err2[n, kb, f] / nrm2[n, kb]))
            for eps in (e, np.nextafter(e, 0.0), np.nextafter(e, 1.0), e * (1 + 3e-6), e * (1 - 3e-6)):
                kw = {key: float(eps)}
                np.testing.assert_array_equal(gpu_plan(W, **kw), orc.plan(W, **kw), err_msg=f"{idx} {kw}")


def test_plan_row_stride(orc):
    """ldw > K: the planner reads W[n, :K] of a wider array."""
    Wide = wl.small_weight(seed=3, n=64, k=384)
    W = gpu(Wide)[:, 64:320]
    fmt = api.plan(W)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fmt.cpu().numpy(), orc.plan(np.ascontiguousarray(Wide[:, 64:320])))


@pytest.mark.parametrize("eps4", [0.04, 0.08, 0.16])
def test_plan_mlp_layer(orc, eps4):
    W = wl.mlp_weight(0, dim=4096)[:1024]
    np.testing.assert_array_equal(gpu_plan(W, eps_int4=eps4), orc.plan(W, eps_int4=eps4))


def test_plan_counts(orc):
    W = edge_matrix(rows=50)
    fmt = api.plan(gpu(W))
    c = api.counts(fmt)
    assert c == list(np.bincount(fmt.cpu().numpy().ravel(), minlength=5))


# ---------------------------------------------------------------------------
# Packer (codes, scales and the whole buffer, byte for byte)
# ---------------------------------------------------------------------------
def gpu_pack_bytes(W, fmt, R):
    pw = api.pack(gpu(W), gpu(fmt), row_tile=R)
    torch.cuda.synchronize()
    return pw.buf.cpu().numpy(), pw


@pytest.mark.parametrize("R", [1, 4, 8, 16])
def test_pack_small_weight(orc, R):
    W = wl.small_weight()
    fmt = orc.plan(W)
    got, _ = gpu_pack_bytes(W, fmt, R)
    np.testing.assert_array_equal(got, orc.pack(W, fmt, R))


@pytest.mark.parametrize("force", [INT4, INT8, BF16, FP16, FP32])
def test_pack_forced_formats(orc, force):
    """Every block in one format: all codes and scales of that format."""
    W = wl.small_weight(seed=1)
    fmt = orc.plan(W, force=force)
    got, _ = gpu_pack_bytes(W, fmt, 16)
    np.testing.assert_array_equal(got, orc.pack(W, fmt, 16))


def test_pack_mixed_random_formats_ragged(orc):
    rng = np.random.default_rng(9)
    W = (rng.normal(size=(37, 320)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(37, 5)).astype(np.uint8)
    for R in (4, 16):
        got, _ = gpu_pack_bytes(W, fmt, R)
        np.testing.assert_array_equal(got, orc.pack(W, fmt, R))


@pytest.mark.parametrize("force", [INT4, INT8, FP32])
def test_pack_edge_blocks(orc, force):
    """Subnormal, huge, tie, NaN and Inf blocks: scales (including the
    canonical NaN / Inf scale) and codes bit-exact."""
    W = edge_matrix()
    fmt = orc.plan(W, force=force)
    got, _ = gpu_pack_bytes(W, fmt, 8)
    np.testing.assert_array_equal(got, orc.pack(W, fmt, 8))


@pytest.mark.parametrize("force", [BF16, FP16])
def test_pack_edge_blocks_16bit(orc, force):
    W = edge_matrix()
    keep = np.all(finite_rows(W), axis=1)
    W = np.ascontiguousarray(W[keep])
    fmt = orc.plan(W, force=force)
    got, _ = gpu_pack_bytes(W, fmt, 8)
    np.testing.assert_array_equal(got, orc.pack(W, fmt, 8))


@pytest.mark.parametrize("N,KB,R,offset", [
    (1030, 272, 16, 0),   # 65 x 272 columns: 70 segments of the index passes, ragged last tile and segment
    (1030, 277, 4, 0),    # 258 x 277 columns: 280 segments, segment edges inside tiles
    (1030, 272, 16, 1),   # map at an address that is not 16-byte aligned
])
def test_pack_index_chunks(orc, N, KB, R, offset):
    """The per-format counts, their scan within 256-column segments and the
    segment offsets over many segments; random formats so every format
    occurs.  (A segment holding 4096 blocks of one format, the largest its
    16-bit fields carry, is in the forced full-layer packs below.)"""
    rng = np.random.default_rng(N + KB + R + offset)
    W = (rng.normal(size=(N, 64 * KB)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(N, KB)).astype(np.uint8)
    raw = torch.zeros(N * KB + 64, dtype=torch.uint8, device=dev())
    fmt_d = raw[offset:offset + N * KB].view(N, KB)
    fmt_d.copy_(gpu(fmt))
    pw = api.pack(gpu(W), fmt_d, row_tile=R)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pw.buf.cpu().numpy(), orc.pack(W, fmt, R))


def test_pack_mlp_layer(orc):
    W = wl.mlp_weight(2, dim=4096)[:512]
    fmt = orc.plan(W)
    got, _ = gpu_pack_bytes(W, fmt, 16)
    np.testing.assert_array_equal(got, orc.pack(W, fmt, 16))


# ---------------------------------------------------------------------------
# Linear
# ---------------------------------------------------------------------------
def run_linear(W, fmt, xbits, R=16, act=0, ldx_pad=0, ldy_pad=0, path=B.HT_PATH_AUTO):
    pw = api.pack(gpu(W), gpu(fmt), row_tile=R)
    M, K = xbits.shape
    xs = torch.zeros((M, K + ldx_pad), dtype=torch.bfloat16, device=dev())
    xs[:, :K] = bf16_gpu(xbits)
    ys = torch.full((M, W.shape[0] + ldy_pad), 7.0, dtype=torch.float32, device=dev())
    x_v, y_v = xs[:, :K], ys[:, :W.shape[0]]
    api.linear(pw, x_v, act=act, out=y_v, path=path)
    torch.cuda.synchronize()
    if ldy_pad:
        assert torch.all(ys[:, W.shape[0]:] == 7.0)   # padding untouched
    return y_v.cpu().numpy()


@pytest.mark.parametrize("path", [B.HT_PATH_GEMV, B.HT_PATH_AUTO])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 13])
def test_linear_small_weight(orc, M, path):
    """The register path at 1 to 13 rows (up to 8 rows per launch, so 13 is
    two launches), and what AUTO picks (the MFMA decode path from 4 rows)."""
    W = wl.small_weight()
    fmt = orc.plan(W)
    x = wl.to_bf16_bits(wl.small_activation(m=M))
    check_close(run_linear(W, fmt, x, path=path), orc.linear(W, fmt, x), f"M={M} path={path}")


@pytest.mark.parametrize("R", [1, 4, 16])
def test_linear_all_formats(orc, R):
    rng = np.random.default_rng(17)
    W = (rng.normal(size=(200, 512)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(200, 8)).astype(np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(3, 512)).astype(np.float32))
    check_close(run_linear(W, fmt, x, R=R), orc.linear(W, fmt, x), f"R={R}")


@pytest.mark.parametrize("force", [INT4, INT8, BF16, FP16, FP32])
def test_linear_single_format(orc, force):
    W = wl.small_weight(seed=4)
    fmt = orc.plan(W, force=force)
    x = wl.to_bf16_bits(wl.small_activation(m=2))
    check_close(run_linear(W, fmt, x), orc.linear(W, fmt, x), f"force={force}")


def test_linear_relu_strides_ragged(orc):
    rng = np.random.default_rng(18)
    W = (rng.normal(size=(37, 192)) * 0.1).astype(np.float32)
    fmt = orc.plan(W, eps_int4=0.2)
    x = wl.to_bf16_bits(rng.normal(size=(4, 192)).astype(np.float32))
    y = run_linear(W, fmt, x, act=1, ldx_pad=64, ldy_pad=5)
    check_close(y, np.maximum(orc.linear(W, fmt, x), 0), "relu/strides")


def test_linear_single_block(orc):
    W = (np.arange(64, dtype=np.float32) - 31.5)[None, :] / 64
    fmt = orc.plan(W)
    x = wl.to_bf16_bits(np.ones((1, 64), np.float32))
    check_close(run_linear(W, fmt, x), orc.linear(W, fmt, x), "1x64")


def test_linear_long_k_split(orc):
    """K = 14336 (the 8B-shaped down projection width): the launch splits K
    and a second kernel adds the splits in order."""
    shp = wl.LinearShape("down", 96, 14336)
    W = wl.llama8b_weight(0, shp)
    fmt = orc.plan(W)
    pw = api.pack(gpu(W), gpu(fmt))
    assert B.ht_linear_workspace(pw.desc, 1) > 0
    for M in (1, 4):
        x = wl.to_bf16_bits(wl.activation("llama8b", M, 14336))
        check_close(run_linear(W, fmt, x), orc.linear(W, fmt, x), f"K=14336 M={M}")


@pytest.mark.parametrize("M", [1, 16, 64])
def test_linear_fused_projections(orc, M):
    """q|k|v rows concatenated into one weight (the fused projection of the
    transformer decode stacks): its plan is the per-part plans stacked (the
    plan is per block), every output matches the oracle, and each part's rows
    equal the separate linear's within fp32 summation order (K-splits and
    paths may differ with the row count): 1e-5 * max|y|."""
    rng = np.random.default_rng(900 + M)
    parts = [(rng.normal(0.0, 0.02, size=(n, 512)) * np.where(rng.random((n, 512)) < 0.001, 30.0, 1.0))
             .astype(np.float32) for n in (256, 64, 64)]
    W = np.concatenate(parts)
    fmt = gpu_plan(W)
    np.testing.assert_array_equal(fmt, np.concatenate([orc.plan(Wp) for Wp in parts]))
    x = wl.to_bf16_bits(rng.normal(size=(M, 512)).astype(np.float32))
    y = run_linear(W, fmt, x)
    check_close(y, orc.linear(W, fmt, x), f"fused M={M}")
    r0 = 0
    for Wp in parts:
        yp = run_linear(Wp, gpu_plan(Wp), x)
        ys = y[:, r0:r0 + Wp.shape[0]]
        assert np.max(np.abs(ys - yp)) <= 1e-5 * max(np.max(np.abs(yp)), 1e-30)
        r0 += Wp.shape[0]


def test_linear_deterministic():
    W = wl.mlp_weight(1, dim=4096)[:2048]
    Wg = gpu(W)
    fmt = api.plan(Wg)
    pw = api.pack(Wg, fmt)
    x = bf16_gpu(wl.to_bf16_bits(wl.mlp_activation(3)))
    y1 = api.linear(pw, x).clone()
    y2 = api.linear(pw, x).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ---------------------------------------------------------------------------
# The 4096-wide, depth-4 MLP at the benchmark's launch configuration
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def mlp4096(orc):
    Ws = [wl.mlp_weight(l) for l in range(wl.MLP_DEPTH)]
    fmts = [orc.plan(W) for W in Ws]
    pws = []
    for W, f in zip(Ws, fmts):
        Wg = gpu(W)
        fg = api.plan(Wg)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(fg.cpu().numpy(), f)   # planner parity at full size
        pws.append(api.pack(Wg, fg, row_tile=16))
        del Wg
    return Ws, fmts, pws


@pytest.mark.parametrize("M,path", [(1, B.HT_PATH_AUTO), (1, B.HT_PATH_GEMV), (2, B.HT_PATH_FUSED),
                                    (3, B.HT_PATH_FUSED), (4, B.HT_PATH_FUSED), (4, B.HT_PATH_GEMV),
                                    (8, B.HT_PATH_AUTO), (16, B.HT_PATH_AUTO), (32, B.HT_PATH_AUTO),
                                    (48, B.HT_PATH_AUTO)])
def test_mlp_teacher_forced(orc, mlp4096, M, path):
    Ws, fmts, pws = mlp4096
    x = wl.to_bf16_bits(wl.mlp_activation(M))
    ws = api.mlp_workspace(pws, M, dev())
    y, dumps = api.mlp(pws, bf16_gpu(x), dump=True, ws=ws, path=path)
    torch.cuda.synchronize()
    assert int(ws[8:12].view(torch.int32).item()) == 0       # no barrier wait expired
    h_in = x
    for l in range(wl.MLP_DEPTH):
        z = orc.linear(Ws[l], fmts[l], h_in)
        if l + 1 < wl.MLP_DEPTH:
            h_gpu = dumps[l].cpu().view(torch.int16).numpy().view(np.uint16)
            hv = wl.bf16_bits_to_f32(h_gpu).astype(np.float64)
            r = np.maximum(z, 0)
            # bf16 output: tolerance plus half a bf16 ulp of the value
            err = np.abs(hv - r) - np.abs(r) * 2.0 ** -8
            assert np.max(err) <= TOL * np.max(r), f"layer {l}"
            h_in = h_gpu
        else:
            check_close(y.cpu().numpy(), np.maximum(z, 0), f"last layer M={M}")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_mlp_fused_equals_per_layer(mlp4096, M):
    """The single persistent launch computes exactly what one launch per
    layer computes (same block partials, same fixed-order row sums), and is
    bitwise reproducible over repeated calls on one workspace."""
    _, _, pws = mlp4096
    x = bf16_gpu(wl.to_bf16_bits(wl.mlp_activation(M, seed=3)))
    ws = api.mlp_workspace(pws, M, dev())
    y_ref = api.mlp(pws, x, ws=ws, path=B.HT_PATH_GEMV).clone()
    for _ in range(3):
        y = api.mlp(pws, x, ws=ws, path=B.HT_PATH_FUSED)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
    assert int(ws[8:12].view(torch.int32).item()) == 0


def test_mlp_fused_ragged_layers(orc):
    """Layers of different widths (tiles per layer differ; workgroups without
    a tile in a layer only take part in its barrier), ragged last tile."""
    rng = np.random.default_rng(71)
    dims = [512, 1024, 256, 200]   # 64, 16 and 13 row tiles; the last one ragged
    Ws = [(rng.standard_t(4, size=(dims[i + 1], dims[i])) * 0.03).astype(np.float32) for i in range(3)]
    fmts = [orc.plan(W) for W in Ws]
    pws = [api.pack(gpu(W), gpu(f)) for W, f in zip(Ws, fmts)]
    x = wl.to_bf16_bits(rng.normal(size=(2, 512)).astype(np.float32))
    ws = api.mlp_workspace(pws, 2, dev())
    y_f, d_f = api.mlp(pws, bf16_gpu(x), dump=True, ws=ws, path=B.HT_PATH_FUSED)
    y_g, d_g = api.mlp(pws, bf16_gpu(x), dump=True, ws=ws, path=B.HT_PATH_GEMV)
    torch.cuda.synchronize()
    assert torch.equal(y_f, y_g)
    for a_, b_ in zip(d_f, d_g):
        assert torch.equal(a_, b_)
    h1 = d_f[-1].cpu().view(torch.int16).numpy().view(np.uint16)
    check_close(y_f.cpu().numpy(), np.maximum(orc.linear(Ws[-1], fmts[-1], h1), 0), "last layer")
    assert int(ws[8:12].view(torch.int32).item()) == 0


def test_mlp_fused_refuses_what_does_not_fit(mlp4096):
    """The single-launch path takes at most 4 rows of x (16-row tiles x 4 rows
    fill the 64-entry LDS row buffer): at M = 5 HT_PATH_FUSED reports
    HT_EINVAL and HT_PATH_AUTO runs one launch per layer."""
    _, _, pws = mlp4096
    x = bf16_gpu(wl.to_bf16_bits(wl.mlp_activation(5)))
    ws = api.mlp_workspace(pws, 5, dev())
    with pytest.raises(B.HTError) as e:
        api.mlp(pws, x, ws=ws, path=B.HT_PATH_FUSED)
    assert e.value.code == 1
    y = api.mlp(pws, x, ws=ws, path=B.HT_PATH_AUTO)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(y))


def test_mlp_end_to_end_info(orc, mlp4096):
    """End to end without teacher forcing (rounding differences of the bf16
    activations compound over layers): reported with a looser bound."""
    Ws, fmts, pws = mlp4096
    x = wl.to_bf16_bits(wl.mlp_activation(1))
    y = api.mlp(pws, bf16_gpu(x))
    torch.cuda.synchronize()
    y_or, _ = orc.mlp(Ws, fmts, x)
    err = np.max(np.abs(y.cpu().numpy() - y_or)) / np.max(np.abs(y_or))
    print(f"MLP end-to-end relative max error {err:.3e}")
    assert err < 2e-2


# ---------------------------------------------------------------------------
# Transformer-shaped layers at full size (sampled outputs)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,name", [("tinyllama", "k"), ("tinyllama", "down"), ("llama8b", "gate"),
                                      ("llama8b", "v"), ("llama8b", "down")])
def test_full_size_layers_sampled(orc, cfg, name):
    shapes = wl.tinyllama_shapes() if cfg == "tinyllama" else wl.llama8b_shapes()
    shp = [s for s in shapes if s.name == name][0]
    W = (wl.tinyllama_weight if cfg == "tinyllama" else wl.llama8b_weight)(0, shp)
    fmt_or = orc.plan(W)
    Wg = gpu(W)
    fmt = api.plan(Wg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fmt.cpu().numpy(), fmt_or)
    pw = api.pack(Wg, fmt)
    x1 = wl.to_bf16_bits(wl.activation(cfg, 1, shp.k))
    y1 = api.linear(pw, bf16_gpu(x1))
    torch.cuda.synchronize()
    check_close(y1.cpu().numpy(), orc.linear(W, fmt_or, x1), f"{cfg}.{name} M=1")
    M = 16
    x = wl.to_bf16_bits(wl.activation(cfg, M, shp.k))
    y = api.linear(pw, bf16_gpu(x))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    mi = rng.integers(0, M, size=128)
    ni = rng.integers(0, shp.n, size=128)
    ys = orc.linear_sampled(W, fmt_or, x, mi, ni)
    # scale: the largest sampled oracle value (a lower bound of max|y|, so
    # the bound is at least as strict as the full-output one)
    assert np.max(np.abs(y.cpu().numpy()[mi, ni] - ys)) <= TOL * np.max(np.abs(ys)), (cfg, name, M)


@pytest.mark.parametrize("M", [4, 2])
def test_register_path_large_lds(orc, M):
    """The register path without a K-split where x plus the block partials
    need more than 64 KiB of LDS: 4 rows over K = 4096 (x alone is exactly
    the 64 KiB limit) and 2 rows over K = 14336."""
    K = 4096 if M == 4 else 14336
    rng = np.random.default_rng(50 + M)
    W = (rng.standard_t(4, size=(512, K)) * 0.02).astype(np.float32)
    fmt = orc.plan(W)
    pw = api.pack(gpu(W), gpu(fmt))
    assert B.ht_linear_workspace(pw.desc, M, B.HT_PATH_GEMV) == 0 or K == 14336
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    y = api.linear(pw, bf16_gpu(x), path=B.HT_PATH_GEMV)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), orc.linear(W, fmt, x), f"M={M} K={K}")


def test_decode_batch4_full_layer(orc):
    """Llama-8B-shaped q projection (4096 x 4096) at batch 4 on the decode
    path, every output against the oracle."""
    shp = [s for s in wl.llama8b_shapes() if s.name == "q"][0]
    W = wl.llama8b_weight(0, shp)
    fmt = orc.plan(W)
    pw = api.pack(gpu(W), gpu(fmt))
    x = wl.to_bf16_bits(wl.activation("llama8b", 4, shp.k, seed=3))
    y = api.linear(pw, bf16_gpu(x))
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), orc.linear(W, fmt, x), "llama8b.q M=4")


@pytest.mark.parametrize("force", [INT4, INT8])
def test_plan_pack_forced_full_layer(orc, force):
    """The planner/packer sweep's reference points at full layer size: every
    block forced to INT4 or INT8 on the 14336 x 4096 gate weight; the map and
    the whole packed buffer byte for byte."""
    shp = [s for s in wl.llama8b_shapes() if s.name == "gate"][0]
    W = wl.llama8b_weight(0, shp)
    fmt = gpu_plan(W, force_format=force)
    np.testing.assert_array_equal(fmt, orc.plan(W, force=force))
    got, _ = gpu_pack_bytes(W, fmt, 16)
    np.testing.assert_array_equal(got, orc.pack(W, fmt, 16))


def _small_stack(orc, dims, seed):
    rng = np.random.default_rng(seed)
    Ws = [(rng.standard_t(4, size=(dims[i + 1], dims[i])) * 0.03).astype(np.float32) for i in range(len(dims) - 1)]
    fmts = [orc.plan(W) for W in Ws]
    return Ws, fmts, [api.pack(gpu(W), gpu(f)) for W, f in zip(Ws, fmts)]


@pytest.mark.parametrize("preset", [0xFFFFFFFE, 14, 0])
def test_mlp_fused_call_counter_cycle(orc, preset):
    """Consecutive single-launch calls on one workspace never share a call
    tag, also across the end of the counter's cycle and from a counter word
    that was not initialised by the library (preset here): three calls with
    different x, each equal bitwise to one launch per layer (which uses no
    tags) and the last layer within the bar of the oracle; no wait expires."""
    Ws, fmts, pws = _small_stack(orc, [512, 512, 512, 256], 81)
    M = 2
    ws = api.mlp_workspace(pws, M, dev())
    ws[0:4].view(torch.int32).fill_(int(np.array(preset, np.uint32).view(np.int32)))
    for call in range(3):
        x = wl.to_bf16_bits(np.random.default_rng(90 + call).normal(size=(M, 512)).astype(np.float32))
        ref = api.mlp(pws, bf16_gpu(x), path=B.HT_PATH_GEMV)
        y, d = api.mlp(pws, bf16_gpu(x), dump=True, ws=ws, path=B.HT_PATH_FUSED)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"call {call} after preset {preset:#x}"
        h1 = d[-1].cpu().view(torch.int16).numpy().view(np.uint16)
        check_close(y.cpu().numpy(), np.maximum(orc.linear(Ws[-1], fmts[-1], h1), 0), f"call {call}")
        assert int(ws[8:12].view(torch.int32).item()) == 0
        assert 0 <= int(ws[0:4].view(torch.int32).item()) < 15      # the counter stays in its cycle


@pytest.mark.parametrize("M", [1, 2, 4])
def test_mlp_fused_uneven_stacks(orc, M):
    """The single launch needs every workgroup to own a row tile of some
    hidden layer (workgroup 0's advance of the call counter is ordered after
    the others' reads only through the hidden layers' words).  256 -> 256 ->
    4096 (16 hidden tiles, 256 in the last layer) is refused by
    HT_PATH_FUSED and runs one launch per layer under HT_PATH_AUTO; 256 ->
    4096 -> 256 -> 4096 runs as one launch although 240 of its workgroups
    own tiles only in the first hidden layer and the last layer: bitwise the
    per-layer result call after call, no wait expires."""
    Ws, fmts, pws = _small_stack(orc, [256, 256, 4096], 83)
    ws = api.mlp_workspace(pws, M, dev())
    x = wl.to_bf16_bits(np.random.default_rng(94).normal(size=(M, 256)).astype(np.float32))
    with pytest.raises(B.HTError) as e:
        api.mlp(pws, bf16_gpu(x), ws=ws, path=B.HT_PATH_FUSED)
    assert e.value.code == 1
    y, d = api.mlp(pws, bf16_gpu(x), dump=True, ws=ws, path=B.HT_PATH_AUTO)
    if M < 4:   # AUTO's per-layer launches are the register path below 4 rows
        assert torch.equal(y, api.mlp(pws, bf16_gpu(x), path=B.HT_PATH_GEMV))
    h1 = d[-1].cpu().view(torch.int16).numpy().view(np.uint16)
    check_close(y.cpu().numpy(), np.maximum(orc.linear(Ws[-1], fmts[-1], h1), 0), "refused stack, last layer")

    Ws, fmts, pws = _small_stack(orc, [256, 4096, 256, 4096], 84)
    ws = api.mlp_workspace(pws, M, dev())
    for call in range(4):
        x = wl.to_bf16_bits(np.random.default_rng(95 + call).normal(size=(M, 256)).astype(np.float32))
        ref = api.mlp(pws, bf16_gpu(x), path=B.HT_PATH_GEMV)
        y, d = api.mlp(pws, bf16_gpu(x), dump=True, ws=ws, path=B.HT_PATH_FUSED)
        torch.cuda.synchronize()
        assert int(ws[8:12].view(torch.int32).item()) == 0, f"call {call}: a wait expired"
        assert torch.equal(y, ref), f"call {call}"
    h2 = d[-1].cpu().view(torch.int16).numpy().view(np.uint16)
    check_close(y.cpu().numpy(), np.maximum(orc.linear(Ws[-1], fmts[-1], h2), 0), "last layer")


def test_pack_full_mlp_layer_natural_plan(orc):
    """The benchmark's own plan and pack: a full 4096 x 4096 MLP layer under
    the default thresholds, map and the whole packed buffer byte for byte."""
    W = wl.mlp_weight(1)
    fmt_or = orc.plan(W)
    Wg = gpu(W)
    fmt = api.plan(Wg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fmt.cpu().numpy(), fmt_or)
    pw = api.pack(Wg, fmt, row_tile=16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pw.buf.cpu().numpy(), orc.pack(W, fmt_or, 16))
