"""GPU parity of the int8 matrix-core path (HT_PATH_GEMM_I8) against the CPU oracle.

A 256-column weight tile whose blocks are all INT8 over a K-split runs on the
int8 matrix cores with x in its two-plane encoding; every other tile runs the
bfloat16 MFMA path.  Checks, on the same seeded inputs:
  * the encoded x the kernel leaves in the workspace is bit-identical to
    oracle.x_planes (white-box: planes in MFMA operand order, row scales);
  * integer tiles match oracle.linear_xplanes (x_hat . W_hat^T in fp64) to
    fp32 rounding (5e-6 of the row's sum of |terms|), and the exact linear
    within the 1e-3 * max|y| bar;
  * the other tiles are bitwise equal to HT_PATH_GEMM's output;
  * K-splits mixing integer and bfloat16 splits, ragged M and N, ReLU,
    all-zero and non-finite rows, run-to-run reproducibility, and the full
    4096 x 4096 layer at 2048 rows (sampled outputs).
"""
import numpy as np
import pytest
import torch

from block_planner_amd import api
from block_planner_amd import binding as B
from block_planner_amd import workloads as wl

pytestmark = pytest.mark.gpu

INT8 = 1
TOL = 1e-3
I8, GEMM = B.HT_PATH_GEMM_I8, B.HT_PATH_GEMM


def dev():
    return torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_gpu(xbits):
    return gpu(xbits.view(np.int16)).view(torch.bfloat16)


def run(pw, xbits, path, act=0, ws_out=None):
    M = xbits.shape[0]
    ws = api.workspace(B.ht_linear_workspace(pw.desc, M, path), dev())
    y = api.linear(pw, bf16_gpu(xbits), act=act, ws=ws, path=path)
    torch.cuda.synchronize()
    if ws_out is not None:
        ws_out.append(ws)
    return y.cpu().numpy().astype(np.float64)


TILE = 256   # weight rows per tile of the int8 path


def int8_tiles(fmt, KBs=None):
    """[NT][S] booleans: 256-row weight tile nt is all INT8 over split s."""
    N, KB = fmt.shape
    KBs = KBs or KB
    S = (KB + KBs - 1) // KBs
    NT = (N + TILE - 1) // TILE
    out = np.zeros((NT, S), bool)
    for nt in range(NT):
        for s in range(S):
            out[nt, s] = np.all(fmt[TILE * nt:TILE * nt + TILE, s * KBs:min(KB, (s + 1) * KBs)] == INT8)
    return out


def splits(pw, M):
    """K-split count and K-blocks per split the MFMA path uses for M rows."""
    KB = pw.K // 64
    ws = B.ht_linear_workspace(pw.desc, M, GEMM)
    S = ws // (M * pw.N * 4) if ws else 1
    KBs = (KB + S - 1) // S
    return (KB + KBs - 1) // KBs, KBs


def expected(orc, W, fmt, xbits, KBs):
    """y with x_hat on the integer (tile, split) pieces and x elsewhere (fp64),
    and sum_k |x . w| per output for the rounding bound."""
    wh = orc.dequant(W, fmt)
    xh = orc.x_hat(*orc.x_planes(xbits))
    x = wl.bf16_bits_to_f32(xbits).astype(np.float64)
    q = int8_tiles(fmt, KBs)
    M, N = xbits.shape[0], W.shape[0]
    y = np.zeros((M, N))
    mag = np.zeros((M, N))
    for nt in range(q.shape[0]):
        cols = slice(TILE * nt, min(N, TILE * nt + TILE))
        for s in range(q.shape[1]):
            ks = slice(64 * s * KBs, min(W.shape[1], 64 * (s + 1) * KBs))
            xs = xh if q[nt, s] else x
            y[:, cols] += xs[:, ks] @ wh[cols, ks].T
            mag[:, cols] += np.abs(xs[:, ks]) @ np.abs(wh[cols, ks]).T
    return y, mag, q


def check(orc, W, fmt, xbits, what, act=0):
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    M = xbits.shape[0]
    S, KBs = splits(pw, M)
    wss = []
    y = run(pw, xbits, I8, act=act, ws_out=wss)
    y_ref, mag, q = expected(orc, W, fmt, xbits, KBs)
    if act:
        y_ref = np.maximum(y_ref, 0.0)
    # fp32 accumulation against the fp64 sum of the same terms
    assert np.all(np.abs(y - y_ref) <= 5e-6 * mag + 1e-30), f"{what}: {np.max(np.abs(y - y_ref) / (mag + 1e-30)):.2e}"
    # and the exact linear within the bar
    y_ex = orc.linear(W, fmt, xbits)
    if act:
        y_ex = np.maximum(y_ex, 0.0)
    err = np.max(np.abs(y - y_ex))
    assert err <= TOL * np.max(np.abs(y_ex)), f"{what}: {err:.3e}"
    # tiles that are not integer over every split equal the bfloat16 MFMA path bitwise
    y_g = run(pw, xbits, GEMM, act=act)
    for nt in range(q.shape[0]):
        if not q[nt].any():
            cols = slice(TILE * nt, min(W.shape[0], TILE * nt + TILE))
            assert np.array_equal(y[:, cols], y_g[:, cols]), f"{what}: tile {nt}"
    return pw, y, q, wss[0], S


def decode_planes(ws, M, K):
    """hi, lo [M][K] and row scales [M] from the workspace (operand order
    [16-row group][kb][plane][lane = row + 16 * (entry / 16)][16 bytes])."""
    G, KB = (M + 15) // 16, K // 64
    raw = ws.cpu().numpy()
    p = raw[:G * KB * 2048].view(np.int8).reshape(G, KB, 2, 4, 16, 16)   # g, kb, plane, quarter, row, byte
    planes = p.transpose(2, 0, 4, 1, 3, 5).reshape(2, G * 16, K)[:, :M]
    off = (G * KB * 2048 + 255) // 256 * 256
    rs = raw[off:off + G * 64].view(np.float32)[:M]
    return planes[0], planes[1], rs


@pytest.mark.parametrize("N,K,M", [(256, 256, 64), (512, 512, 300), (600, 1024, 130), (72, 256, 5), (4096, 4096, 16)])
def test_i8_all_int8(orc, N, K, M):
    rng = np.random.default_rng(N + K + M)
    W = (rng.standard_t(4, size=(N, K)) * 0.02).astype(np.float32)
    fmt = np.full((N, K // 64), INT8, np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32) * np.float32(2.0))
    _, _, q, ws, _ = check(orc, W, fmt, x, f"{N}x{K} M={M}")
    assert q.all()
    hi, lo, rs = decode_planes(ws, M, K)
    h_o, l_o, se = orc.x_planes(x)
    assert np.array_equal(hi, h_o) and np.array_equal(lo, l_o)
    assert np.array_equal(rs.astype(np.float64), np.ldexp(1.0, se))


def test_i8_mixed_tiles(orc):
    """Tiles 0 and 2 all INT8 (the last one ragged), tile 1 mixed: both
    kernels in one call."""
    rng = np.random.default_rng(41)
    N, K, M = 700, 768, 260
    W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(N, K // 64)).astype(np.uint8)
    fmt[0:256] = INT8
    fmt[512:] = INT8
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    _, _, q, _, _ = check(orc, W, fmt, x, "mixed", act=B.HT_ACT_RELU)
    assert q[:, 0].tolist() == [True, False, True]


def test_i8_split_mixes_paths(orc):
    """Few output tiles: K is split, and tile 0 is INT8 only in the first
    half of K, so its splits go to different kernels."""
    rng = np.random.default_rng(43)
    N, K, M = 768, 8192, 24
    W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
    fmt = rng.choice(np.array([1, 1, 1, 4], np.uint8), size=(N, K // 64))
    fmt[0:256, :64] = INT8
    fmt[512:768] = INT8
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    _, _, q, _, S = check(orc, W, fmt, x, "split")
    assert S > 1 and q[0].any() and not q[0].all() and q[2].all()


def test_i8_special_rows(orc):
    """An all-zero row gives zeros, a row holding Inf gives NaN on the
    integer tiles, the other rows are unaffected."""
    rng = np.random.default_rng(44)
    N, K, M = 128, 512, 40
    W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
    fmt = np.full((N, K // 64), INT8, np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    x[3] = 0
    x[7, 100] = 0x7F80            # +Inf
    x[9, 5] = 0xFF80              # -Inf
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    y = run(pw, x, I8)
    assert np.all(y[3] == 0.0)
    assert np.all(np.isnan(y[7])) and np.all(np.isnan(y[9]))
    ok = np.setdiff1d(np.arange(M), [7, 9])
    y_ref = orc.linear_xplanes(W, fmt, x[ok])
    mag = np.abs(orc.x_hat(*orc.x_planes(x[ok]))) @ np.abs(orc.dequant(W, fmt)).T
    assert np.all(np.abs(y[ok] - y_ref) <= 5e-6 * mag + 1e-30)


def test_i8_benchmark_mix_is_gemm(orc):
    """On planned Llama-shaped weights no 64-column tile is all INT8, and the
    path's output is the bfloat16 MFMA path's, bitwise."""
    shp = [s for s in wl.llama8b_shapes() if s.name == "k"][0]
    W = wl.llama8b_weight(0, shp)[:512, :2048]
    fmt = orc.plan(W)
    assert not int8_tiles(fmt).any()
    x = wl.to_bf16_bits(wl.small_activation(m=96, k=2048))
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    assert np.array_equal(run(pw, x, I8), run(pw, x, GEMM))


def test_i8_reproducible():
    rng = np.random.default_rng(45)
    W = (rng.normal(size=(512, 2048)) * 0.05).astype(np.float32)
    fmt = np.full((512, 32), INT8, np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(700, 2048)).astype(np.float32))
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    assert np.array_equal(run(pw, x, I8), run(pw, x, I8))


def test_i8_full_layer_sampled(orc):
    """The Llama q shape (4096 x 4096, every block INT8) at 2048 rows, as
    timed: sampled outputs against x_hat . W_hat^T and the exact linear."""
    shp = [s for s in wl.llama8b_shapes() if s.name == "q"][0]
    W = wl.llama8b_weight(0, shp)
    N, K = W.shape
    fmt = np.full((N, K // 64), INT8, np.uint8)
    M = 2048
    rng = np.random.default_rng(46)
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    y = run(pw, x, I8)
    mi = rng.integers(0, M, size=300)
    ni = rng.integers(0, N, size=300)
    rows = np.unique(mi)
    xh = dict(zip(rows, orc.x_hat(*orc.x_planes(x[rows]))))
    wrows = np.unique(ni)
    wh = dict(zip(wrows, orc.dequant(W[wrows], fmt[wrows])))
    for m, n in zip(mi, ni):
        ref = float(xh[m] @ wh[n])
        mag = float(np.abs(xh[m]) @ np.abs(wh[n]))
        assert abs(y[m, n] - ref) <= 5e-6 * mag, (m, n)
    y_ex = orc.linear_sampled(W, fmt, x, mi, ni)
    assert np.max(np.abs(y[mi, ni] - y_ex)) <= TOL * np.max(np.abs(y_ex))


def test_i8_too_few_int8_blocks_is_gemm(orc):
    """Fewer INT8 blocks than one tile needs: the call is the bfloat16 MFMA
    path's alone (same workspace, bitwise the same output)."""
    rng = np.random.default_rng(47)
    N, K, M = 512, 1024, 200
    W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
    fmt = rng.choice(np.array([2, 3, 4], np.uint8), size=(N, K // 64))
    fmt[5, 3] = fmt[300, 0] = fmt[511, 15] = INT8
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    assert B.ht_linear_workspace(pw.desc, M, I8) == B.ht_linear_workspace(pw.desc, M, GEMM)
    y = run(pw, x, I8)
    assert np.array_equal(y, run(pw, x, GEMM))
    assert np.max(np.abs(y - orc.linear(W, fmt, x))) <= TOL * np.max(np.abs(orc.linear(W, fmt, x)))


def test_i8_strides_and_tiny(orc):
    """Row strides on x and y (the padding of y untouched), a weight narrower
    than one row tile, and a single row of x."""
    rng = np.random.default_rng(48)
    for N, K, M in ((8, 192, 1), (40, 512, 37)):
        W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
        fmt = np.full((N, K // 64), INT8, np.uint8)
        x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
        pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
        xs = torch.zeros((M, K + 24), dtype=torch.bfloat16, device=dev())
        xs[:, :K] = bf16_gpu(x)
        ys = torch.full((M, N + 12), 7.0, dtype=torch.float32, device=dev())
        ws = api.workspace(B.ht_linear_workspace(pw.desc, M, I8), dev())
        api.linear(pw, xs[:, :K], out=ys[:, :N], ws=ws, path=I8)
        torch.cuda.synchronize()
        assert torch.all(ys[:, N:] == 7.0)
        y = ys[:, :N].cpu().numpy().astype(np.float64)
        y_ref = orc.linear_xplanes(W, fmt, x)
        mag = np.abs(orc.x_hat(*orc.x_planes(x))) @ np.abs(orc.dequant(W, fmt)).T
        assert np.all(np.abs(y - y_ref) <= 5e-6 * mag + 1e-30), (N, K, M)
