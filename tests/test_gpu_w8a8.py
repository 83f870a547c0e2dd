"""GPU parity of the opt-in W8A8 mode (HT_PATH_W8A8) against the CPU oracle.

The mode runs the int8 matrix-core path's tiles (256-column weight tiles whose
blocks are all INT8 over a K-split) with x encoded per token and 64-wide
K-block as one int8 plane and a power-of-two scale (oracle.x_w8a8); every
other tile runs the bfloat16 MFMA path.  Checks, on the same seeded inputs:
  * the encoded x the kernels leave in the workspace is bit-identical to
    oracle.x_w8a8 (codes in MFMA operand order, block scales 2^bexp);
  * integer tiles match oracle.linear_w8a8 (x_hat . W_hat^T in fp64) to fp32
    rounding: 5e-6 of each output's sum of |terms|;
  * the other tiles are bitwise equal to HT_PATH_GEMM's output;
  * K-splits mixing integer and bfloat16 splits, ragged M and N, ReLU,
    all-zero and non-finite blocks, run-to-run reproducibility, strides, and
    the Llama-8B q shape at 2048 rows (sampled outputs).
The mode is a different output function: it is not held to the bf16 bar
against the exact linear (its x has 8 bits per block maximum).
"""
import numpy as np
import pytest
import torch

from block_planner_amd import api
from block_planner_amd import binding as B
from block_planner_amd import workloads as wl

pytestmark = pytest.mark.gpu

INT8 = 1
W8, GEMM = B.HT_PATH_W8A8, B.HT_PATH_GEMM
TILE = 256
XEXP_NONFINITE = -1000


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


def int8_tiles(fmt, KBs):
    N, KB = fmt.shape
    S = (KB + KBs - 1) // KBs
    NT = (N + TILE - 1) // TILE
    out = np.zeros((NT, S), bool)
    for nt in range(NT):
        for s in range(S):
            out[nt, s] = np.all(fmt[TILE * nt:TILE * nt + TILE, s * KBs:min(KB, (s + 1) * KBs)] == INT8)
    return out


def splits(pw, M):
    KB = pw.K // 64
    ws = B.ht_linear_workspace(pw.desc, M, GEMM)
    S = ws // (M * pw.N * 4) if ws else 1
    KBs = (KB + S - 1) // S
    return (KB + KBs - 1) // KBs, KBs


def expected(orc, W, fmt, xbits, KBs):
    """y with the W8A8 x_hat on the integer (tile, split) pieces and x
    elsewhere (fp64), and sum_k |x . w| per output for the rounding bound."""
    wh = orc.dequant(W, fmt)
    xh = orc.x_hat_w8a8(*orc.x_w8a8(xbits))
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
    y = run(pw, xbits, W8, act=act, ws_out=wss)
    y_ref, mag, q = expected(orc, W, fmt, xbits, KBs)
    if act:
        y_ref = np.maximum(y_ref, 0.0)
    assert np.all(np.abs(y - y_ref) <= 5e-6 * mag + 1e-30), f"{what}: {np.max(np.abs(y - y_ref) / (mag + 1e-30)):.2e}"
    y_g = run(pw, xbits, GEMM, act=act)
    for nt in range(q.shape[0]):
        if not q[nt].any():
            cols = slice(TILE * nt, min(W.shape[0], TILE * nt + TILE))
            assert np.array_equal(y[:, cols], y_g[:, cols]), f"{what}: tile {nt}"
    return pw, y, q, wss[0], S


def decode_ws(ws, M, K):
    """codes [M][K] and block scales [M][K/64] from the workspace (codes in
    operand order [16-row group][kb][lane = row + 16 * (entry / 16)][16
    bytes], then the scales [kb][16 * groups])."""
    G, KB = (M + 15) // 16, K // 64
    raw = ws.cpu().numpy()
    c = raw[:G * KB * 1024].view(np.int8).reshape(G, KB, 4, 16, 16)   # g, kb, quarter, row, byte
    codes = c.transpose(0, 3, 1, 2, 4).reshape(G * 16, K)[:M]
    off = (G * KB * 1024 + 255) // 256 * 256
    sx = raw[off:off + KB * G * 16 * 4].view(np.float32).reshape(KB, G * 16)[:, :M].T
    return codes, sx


def scales_of(bexp):
    out = np.ldexp(1.0, np.where(bexp == XEXP_NONFINITE, 0, bexp))
    out[bexp == XEXP_NONFINITE] = np.nan
    return out


@pytest.mark.parametrize("N,K,M", [(256, 256, 64), (512, 512, 300), (600, 1024, 130), (72, 256, 5), (4096, 4096, 16)])
def test_w8a8_all_int8(orc, N, K, M):
    rng = np.random.default_rng(500 + N + K + M)
    W = (rng.standard_t(4, size=(N, K)) * 0.02).astype(np.float32)
    fmt = np.full((N, K // 64), INT8, np.uint8)
    # each K-block of each token with its own magnitude
    mags = np.exp(rng.uniform(-6, 6, size=(M, K // 64))).astype(np.float32)
    x = rng.normal(size=(M, K)).astype(np.float32) * np.repeat(mags, 64, axis=1)
    xb = wl.to_bf16_bits(x)
    _, _, q, ws, _ = check(orc, W, fmt, xb, f"{N}x{K} M={M}")
    assert q.all()
    codes, sx = decode_ws(ws, M, K)
    q_o, bexp = orc.x_w8a8(xb)
    assert np.array_equal(codes, q_o)
    assert np.array_equal(sx.astype(np.float64), scales_of(bexp))


def test_w8a8_mixed_tiles(orc):
    """Tiles 0 and 2 all INT8 (the last one ragged), tile 1 mixed: both
    kernels in one call, with ReLU."""
    rng = np.random.default_rng(541)
    N, K, M = 700, 768, 260
    W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(N, K // 64)).astype(np.uint8)
    fmt[0:256] = INT8
    fmt[512:] = INT8
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    _, _, q, _, _ = check(orc, W, fmt, x, "mixed", act=B.HT_ACT_RELU)
    assert q[:, 0].tolist() == [True, False, True]


def test_w8a8_split_mixes_paths(orc):
    """Few output tiles: K is split, and tile 0 is INT8 only in the first
    half of K, so its splits go to different kernels."""
    rng = np.random.default_rng(543)
    N, K, M = 768, 8192, 24
    W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
    fmt = rng.choice(np.array([1, 1, 1, 4], np.uint8), size=(N, K // 64))
    fmt[0:256, :64] = INT8
    fmt[512:768] = INT8
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    _, _, q, _, S = check(orc, W, fmt, x, "split")
    assert S > 1 and q[0].any() and not q[0].all() and q[2].all()


def test_w8a8_special_blocks(orc):
    """An all-zero token gives zeros; a block holding Inf (or NaN) makes its
    token's outputs NaN; the other tokens are unaffected."""
    rng = np.random.default_rng(544)
    N, K, M = 128, 512, 40
    W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
    fmt = np.full((N, K // 64), INT8, np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    x[3] = 0
    x[7, 100] = 0x7F80            # +Inf
    x[9, 5] = 0x7FC0              # NaN
    x[11, 64:128] = 0             # one all-zero block
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    y = run(pw, x, W8)
    assert np.all(y[3] == 0.0)
    assert np.all(np.isnan(y[7])) and np.all(np.isnan(y[9]))
    ok = np.setdiff1d(np.arange(M), [7, 9])
    y_ref = orc.linear_w8a8(W, fmt, x[ok])
    mag = np.abs(orc.x_hat_w8a8(*orc.x_w8a8(x[ok]))) @ np.abs(orc.dequant(W, fmt)).T
    assert np.all(np.abs(y[ok] - y_ref) <= 5e-6 * mag + 1e-30)


def test_w8a8_reproducible_and_strides(orc):
    rng = np.random.default_rng(545)
    W = (rng.normal(size=(512, 2048)) * 0.05).astype(np.float32)
    fmt = np.full((512, 32), INT8, np.uint8)
    x = wl.to_bf16_bits(rng.normal(size=(700, 2048)).astype(np.float32))
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    assert np.array_equal(run(pw, x, W8), run(pw, x, W8))
    for N, K, M in ((8, 192, 1), (40, 512, 37)):
        W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
        fmt = np.full((N, K // 64), INT8, np.uint8)
        x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
        pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
        xs = torch.zeros((M, K + 24), dtype=torch.bfloat16, device=dev())
        xs[:, :K] = bf16_gpu(x)
        ys = torch.full((M, N + 12), 7.0, dtype=torch.float32, device=dev())
        ws = api.workspace(B.ht_linear_workspace(pw.desc, M, W8), dev())
        api.linear(pw, xs[:, :K], out=ys[:, :N], ws=ws, path=W8)
        torch.cuda.synchronize()
        assert torch.all(ys[:, N:] == 7.0)
        y = ys[:, :N].cpu().numpy().astype(np.float64)
        y_ref = orc.linear_w8a8(W, fmt, x)
        mag = np.abs(orc.x_hat_w8a8(*orc.x_w8a8(x))) @ np.abs(orc.dequant(W, fmt)).T
        assert np.all(np.abs(y - y_ref) <= 5e-6 * mag + 1e-30), (N, K, M)


def test_w8a8_planned_llama_is_gemm(orc):
    """On planned Llama-shaped weights no tile is all INT8: the mode's output
    is the bfloat16 MFMA path's, bitwise."""
    shp = [s for s in wl.llama8b_shapes() if s.name == "k"][0]
    W = wl.llama8b_weight(0, shp)[:512, :2048]
    fmt = orc.plan(W)
    x = wl.to_bf16_bits(wl.small_activation(m=96, k=2048))
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    assert np.array_equal(run(pw, x, W8), run(pw, x, GEMM))


def test_w8a8_full_layer_sampled(orc):
    """The Llama q shape (4096 x 4096, every block INT8) at 2048 rows:
    sampled outputs against x_hat . W_hat^T."""
    shp = [s for s in wl.llama8b_shapes() if s.name == "q"][0]
    W = wl.llama8b_weight(0, shp)
    N, K = W.shape
    fmt = np.full((N, K // 64), INT8, np.uint8)
    M = 2048
    rng = np.random.default_rng(546)
    x = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    pw = api.pack(gpu(W), gpu(fmt), row_tile=16)
    y = run(pw, x, W8)
    mi = rng.integers(0, M, size=300)
    ni = rng.integers(0, N, size=300)
    rows = np.unique(mi)
    xh = dict(zip(rows, orc.x_hat_w8a8(*orc.x_w8a8(x[rows]))))
    wrows = np.unique(ni)
    wh = dict(zip(wrows, orc.dequant(W[wrows], fmt[wrows])))
    for m, n in zip(mi, ni):
        ref = float(xh[m] @ wh[n])
        mag = float(np.abs(xh[m]) @ np.abs(wh[n]))
        assert abs(y[m, n] - ref) <= 5e-6 * mag, (m, n)
