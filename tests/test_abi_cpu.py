"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and its host-side checks reject bad arguments before any launch
(only invalid calls are made here, so nothing reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

from block_planner_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "ht.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ht_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    syms = header_symbols()
    assert len(syms) >= 10
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(B.EXPORTS)


def test_status_strings_and_defaults():
    assert B.ht_status_string(0) == "ok"
    for c in range(1, 6):
        assert B.ht_status_string(c) not in ("ok", "unknown status")
    assert B.ht_status_string(99) == "unknown status"
    p = B.ht_plan_params_default()
    assert (p.eps_int4, p.eps_int8, p.eps_bf16, p.eps_fp16, p.prefer_bf16, p.force_format) == \
        (0.08, 0.01, 0.0, 0.0, 1, -1)


def test_pack_bytes_matches_layout(orc):
    for (N, K, R, c) in [(256, 256, 16, [10, 500, 3, 1, 510]), (37, 192, 16, [20, 20, 20, 20, 31]),
                         (4096, 4096, 16, [163, 195780, 0, 0, 66201]), (256, 2048, 1, [0, 8192, 0, 0, 0]),
                         (5632, 2048, 8, [0, 0, 0, 0, 5632 * 32])]:
        assert B.ht_pack_bytes(N, K, R, c) == orc.pack_layout(N, K, R, c)[0]


@pytest.mark.parametrize("args,code", [
    ((256, 100, 16, [0, 0, 0, 0, 0]), 2),          # K % 64
    ((256, 256, 3, [0, 1024, 0, 0, 0]), 2),        # row tile not a power of two <= 16
    ((256, 256, 32, [0, 1024, 0, 0, 0]), 2),
    ((256, 256, 16, [0, 1000, 0, 0, 0]), 1),       # counts do not sum to N*K/64
    ((256, 256, 16, [-1, 1025, 0, 0, 0]), 1),
    ((0, 256, 16, [0, 0, 0, 0, 0]), 2),
    ((16, 64 * 5000, 16, [0, 80000, 0, 0, 0]), 2), # K/64 * R > 65536 (16-bit block ids)
    ((32768, 32768, 16, [0, 0, 0, 0, 32768 * 512]), 2),  # 4 GiB of FP32 blocks: past 32-bit offsets
])
def test_pack_bytes_rejects(args, code):
    with pytest.raises(B.HTError) as e:
        B.ht_pack_bytes(*args)
    assert e.value.code == code


def _plan_raw(W, N, K, ldw, params, fmt):
    lib = B.load()
    pp = ctypes.byref(params) if params is not None else None
    return lib.ht_plan(W, N, K, ldw, pp, fmt, None)


def test_plan_argument_checks():
    good = 0x10000
    assert _plan_raw(None, 4, 64, 64, None, good) == 1
    assert _plan_raw(good, 4, 64, 64, None, None) == 1
    assert _plan_raw(good, 0, 64, 64, None, good) == 2
    assert _plan_raw(good, 4, 65, 65, None, good) == 2
    assert _plan_raw(good, 4, 128, 64, None, good) == 2          # ldw < K
    assert _plan_raw(good + 4, 4, 64, 64, None, good) == 3       # W misaligned
    assert _plan_raw(good, 4, 64, 66, None, good) == 3           # ldw not a multiple of 4
    for bad in (-0.1, float("nan"), float("inf")):
        p = B.ht_plan_params_default()
        p.eps_int8 = bad
        assert _plan_raw(good, 4, 64, 64, p, good) == 1
    p = B.ht_plan_params_default()
    p.force_format = 5
    assert _plan_raw(good, 4, 64, 64, p, good) == 1
    p.force_format = -2
    assert _plan_raw(good, 4, 64, 64, p, good) == 1


def test_plan_counts_argument_checks():
    lib = B.load()
    assert lib.ht_plan_counts(None, 4, 64, 0x10000, None) == 1
    assert lib.ht_plan_counts(0x10000, 4, 64, None, None) == 1
    assert lib.ht_plan_counts(0x10000, 4, 60, 0x10000, None) == 2
    assert lib.ht_plan_counts(0x10000, 4, 64, 0x10004, None) == 3


def _desc(N=256, K=256, R=16, base=0x100000, counts=None):
    """A descriptor consistent with the layout of (N, K, R, counts) (by
    default every block INT8), offsets from the oracle's own layout
    function; no buffer behind it."""
    import oracle
    d = B.PackedWeight()
    d.N, d.K, d.row_tile, d.n_tiles = N, K, R, (N + R - 1) // R
    counts = [0, N * (K // 64), 0, 0, 0] if counts is None else counts
    size, offs = oracle.pack_layout(N, K, R, counts)
    for f in range(5):
        d.counts[f] = counts[f]
        d.off_ids[f] = offs[1 + f]
        d.off_payload[f] = offs[8 + f]
    d.off_kbidx = offs[0]
    d.off_scale[0], d.off_scale[1] = offs[6], offs[7]
    d.bytes = size
    d.layout_version = 1
    d.base = base
    return d


def _with_counts(d, counts):
    return _desc(int(d.N), int(d.K), int(d.row_tile), d.base, counts)


def test_linear_argument_checks():
    lib = B.load()
    d = _desc()
    x, y = 0x200000, 0x300000
    f = lib.ht_linear_forward
    assert f(None, x, 1, 256, y, 256, 0, 0, None, 0, None) == 1
    bad = _desc()
    bad.layout_version = 7
    assert f(ctypes.byref(bad), x, 1, 256, y, 256, 0, 0, None, 0, None) == 1
    assert f(ctypes.byref(d), None, 1, 256, y, 256, 0, 0, None, 0, None) == 1
    assert f(ctypes.byref(d), x, 1, 256, y, 256, 2, 0, None, 0, None) == 1      # act
    assert f(ctypes.byref(d), x, 1, 256, y, 256, 0, 9, None, 0, None) == 1      # path
    assert f(ctypes.byref(d), x, 0, 256, y, 256, 0, 0, None, 0, None) == 2      # M
    assert f(ctypes.byref(d), x, 1, 128, y, 256, 0, 0, None, 0, None) == 2      # ldx < K
    assert f(ctypes.byref(d), x, 1, 256, y, 100, 0, 0, None, 0, None) == 2      # ldy < N
    assert f(ctypes.byref(d), x + 2, 1, 256, y, 256, 0, 0, None, 0, None) == 3  # x misaligned
    assert f(ctypes.byref(d), x, 1, 260, y, 256, 0, 0, None, 0, None) == 3      # ldx % 8
    big = _desc(N=256, K=64 * 1024, R=16)
    need = B.ht_linear_workspace(big, 1)
    assert need > 0                                                            # needs a K-split
    assert f(ctypes.byref(big), x, 1, 64 * 1024, y, 256, 0, 0, None, 0, None) == 4
    # the MFMA path splits K when it has few output tiles: [S][M][N] fp32
    # partials with 2 <= S <= K/64/4 (at least 4 K-blocks per split)
    for M, path in ((1, B.HT_PATH_GEMM), (16, B.HT_PATH_AUTO), (20, B.HT_PATH_GEMV_MFMA)):
        ws = B.ht_linear_workspace(big, M, path)
        assert ws % (M * 256 * 4) == 0 and 2 <= ws // (M * 256 * 4) <= 1024 // 4
    # the MFMA decode path: 32 rows per launch (partials sized for 32 at
    # most), no split with enough row tiles, row tile 16 only
    assert B.ht_linear_workspace(big, 64, B.HT_PATH_GEMV_MFMA) == B.ht_linear_workspace(big, 32, B.HT_PATH_GEMV_MFMA)
    assert B.ht_linear_workspace(_desc(N=4096, K=4096, R=16), 32, B.HT_PATH_GEMV_MFMA) == 0
    for R in (1, 2, 4, 8):
        with pytest.raises(B.HTError):
            B.ht_linear_workspace(_desc(N=256, K=4096, R=R), 8, B.HT_PATH_GEMV_MFMA)
        assert f(ctypes.byref(_desc(R=R)), x, 8, 256, y, 256, 0, B.HT_PATH_GEMV_MFMA, None, 0, None) == 1
    wide = _desc(N=16384, K=4096, R=16)
    # the int8 matrix-core path, 8192 rows per launch (sized for 8192 at most),
    # decided by the weight's INT8 count: none (too few for any 256-row tile)
    # -> exactly the single-pass MFMA kernel's partials (the MFMA path's
    # workspace below 1024 rows); mixed -> x's two int8 planes
    # (2 bytes per entry, rows in groups of 16) and 16 fp32 row scales per
    # group, each region 256-byte aligned, then the MFMA path's partials; all
    # INT8 -> planes, scales and partials for the int8 kernel's own K-splits
    # (128 x 256 tiles, split when fewer than 192, at least 8 K-blocks each)
    def a256(v):
        return (v + 255) // 256 * 256

    def single_pass_ws(dsc, Mt):
        """K-split partials of the single-pass MFMA kernel (256 x 128 tiles
        from 256 rows), which the int8 path runs beside the int8 kernel."""
        KB = dsc.K // 64
        BM = 256 if Mt >= 256 else 128 if Mt >= 128 else 64
        tiles = (dsc.N + 127) // 128 * ((Mt + BM - 1) // BM)
        if tiles * 4 >= 3 * 256 or KB < 16:
            return 0
        S = min(-(-256 // tiles), KB // 8)
        KBs = -(-KB // S)
        return -(-KB // KBs) * Mt * dsc.N * 4
    for dsc, M in ((wide, 2048), (wide, 20000), (big, 1), (big, 33)):
        Mt = min(M, 8192)
        G, KB = (Mt + 15) // 16, dsc.K // 64
        extra = a256(G * KB * 2048) + a256(G * 16 * 4)
        dsc = _with_counts(dsc, [0, 0, 0, 0, dsc.N * KB])
        assert B.ht_linear_workspace(dsc, M, B.HT_PATH_GEMM_I8) == single_pass_ws(dsc, Mt)
        if M < 1024:
            assert single_pass_ws(dsc, Mt) == B.ht_linear_workspace(dsc, Mt, B.HT_PATH_GEMM)
        dsc = _with_counts(dsc, [0, dsc.N * KB - 1, 0, 0, 1])
        assert B.ht_linear_workspace(dsc, M, B.HT_PATH_GEMM_I8) == extra + single_pass_ws(dsc, Mt)
        dsc = _with_counts(dsc, [0, dsc.N * KB, 0, 0, 0])
        tiles = (Mt + 127) // 128 * ((dsc.N + 255) // 256)
        S = 1
        if tiles * 4 < 3 * 256 and KB >= 16:
            S = min(-(-256 // tiles), KB // 8)
            KBs = -(-KB // S)
            S = -(-KB // KBs)
        assert B.ht_linear_workspace(dsc, M, B.HT_PATH_GEMM_I8) == extra + (S * Mt * dsc.N * 4 if S > 1 else 0)
        # the W8A8 mode: the same tiles and splits, x as one int8 plane (1 byte
        # per entry) and an fp32 scale per row and K-block ([kb][16 * groups])
        extra8 = a256(G * KB * 1024) + a256(KB * G * 16 * 4)
        assert B.ht_linear_workspace(dsc, M, B.HT_PATH_W8A8) == extra8 + (S * Mt * dsc.N * 4 if S > 1 else 0)
        dsc = _with_counts(dsc, [0, dsc.N * KB - 1, 0, 0, 1])
        assert B.ht_linear_workspace(dsc, M, B.HT_PATH_W8A8) == extra8 + single_pass_ws(dsc, Mt)
    for R in (1, 2, 4, 8):
        for path in (B.HT_PATH_GEMM_I8, B.HT_PATH_W8A8):
            with pytest.raises(B.HTError):
                B.ht_linear_workspace(_desc(N=256, K=4096, R=R), 64, path)
            assert f(ctypes.byref(_desc(R=R)), x, 64, 256, y, 256, 0, path, None, 0, None) == 1
    with pytest.raises(B.HTError):
        B.ht_linear_workspace(big, 1, 7)                                        # no such path
    # AUTO on a row tile other than 16 keeps to the other two paths
    assert B.ht_linear_workspace(_desc(N=256, K=64 * 1024, R=8), 8, B.HT_PATH_AUTO) == \
        B.ht_linear_workspace(_desc(N=256, K=64 * 1024, R=8), 8, B.HT_PATH_GEMV)
    # the MFMA path: no K-split with 128 output tiles at 1000 rows; from 1024
    # rows (at least 192 tiles of 256 x 128) it prefers the two-pass kernel,
    # whose workspace holds a 33 KiB record per 128-column x 64-K weight tile
    assert B.ht_linear_workspace(wide, 1000, B.HT_PATH_GEMM) == 0
    assert B.ht_linear_workspace(wide, 2048, B.HT_PATH_GEMM) == (16384 // 128) * (4096 // 64) * 33 * 1024
    assert B.ht_linear_workspace(_desc(N=6144, K=4096, R=16), 1024, B.HT_PATH_GEMM) == 48 * 64 * 33 * 1024
    # 112 x 8 = 896 output tiles: the last round's 128 tiles (half of 256
    # compute units) run as two K halves, whose fp32 partial sums follow the
    # records
    assert B.ht_linear_workspace(_desc(N=14336, K=4096, R=16), 2048, B.HT_PATH_GEMM) == \
        112 * 64 * 33 * 1024 + 128 * 2 * 256 * 128 * 4
    # 188 tiles: the single-pass kernel, which splits K in two below 192
    assert B.ht_linear_workspace(_desc(N=6016, K=4096, R=16), 1024, B.HT_PATH_GEMM) == 2 * 1024 * 6016 * 4
    with pytest.raises(B.HTError):
        B.ht_linear_workspace(big, 1, B.HT_PATH_FUSED)                        # MLP-only path
    assert f(ctypes.byref(d), x, 1, 256, y, 256, 0, B.HT_PATH_FUSED, None, 0, None) == 1


def test_mlp_argument_checks():
    lib = B.load()
    a, b = _desc(256, 256), _desc(128, 512)
    arr = (ctypes.POINTER(B.PackedWeight) * 2)(ctypes.pointer(a), ctypes.pointer(b))
    out = ctypes.c_size_t(0)
    assert lib.ht_mlp_workspace(arr, 2, 1, ctypes.byref(out)) == 2            # K of layer 1 != N of layer 0
    c = _desc(128, 256)
    arr = (ctypes.POINTER(B.PackedWeight) * 2)(ctypes.pointer(a), ctypes.pointer(c))
    assert lib.ht_mlp_workspace(arr, 2, 1, ctypes.byref(out)) == 0
    assert out.value > 0
    assert lib.ht_mlp_forward(arr, 2, 0x200000, 1, 256, 0x300000, 128, None, 0, None, 0, None) == 4
    assert lib.ht_mlp_forward(arr, 2, 0x200000, 1, 256, 0x300000, 128, None, 7, 0x400000, 1 << 20, None) == 1
    assert lib.ht_mlp_forward(arr, 0, 0x200000, 1, 256, 0x300000, 128, None, 0, None, 0, None) == 1
    assert lib.ht_workspace_init(None, 256, None) == 1
    assert lib.ht_workspace_init(0x400004, 256, None) == 3


def test_backward_argument_checks():
    lib = B.load()
    d = _desc(N=256, K=512)
    out = ctypes.c_size_t(0)
    assert lib.ht_linear_backward_workspace(ctypes.byref(d), 0, ctypes.byref(out)) == 2          # M <= 0
    assert lib.ht_linear_backward_workspace(ctypes.byref(_desc(R=8)), 1, ctypes.byref(out)) == 1   # row tile 8
    assert lib.ht_linear_backward_workspace(ctypes.byref(d), 3, ctypes.byref(out)) == 0
    # 16 row tiles: at most 4 tile groups of at least 4 tiles -> [G][min(M, 4)][K] fp32 partials
    assert out.value == 4 * 3 * 512 * 4
    f = lib.ht_linear_backward_data
    dy, dx = 0x200000, 0x300000
    assert f(ctypes.byref(d), dy, 3, 255, dx, 512, None, 0, None) == 2       # lddy < N
    assert f(ctypes.byref(d), dy, 3, 256, dx, 511, None, 0, None) == 2       # lddx < K
    assert f(ctypes.byref(d), dy + 4, 3, 256, dx, 512, None, 0, None) == 3   # misaligned dy
    assert f(ctypes.byref(d), dy, 3, 256, dx, 512, None, 0, None) == 4       # workspace missing
    assert f(ctypes.byref(d), None, 3, 256, dx, 512, None, 0, None) == 1


def test_packed_buffers_stay_below_4gib():
    """The kernels address the packed buffer with 32-bit offsets (buffer
    loads, whose out-of-range offset reads zeros), so the layout refuses a
    buffer of 4 GiB or more: a 65536 x 65536 all-INT8 weight (about 4.8 GB
    packed) is refused by every entry point that takes a descriptor, while
    32768 x 65536 (2.4 GB) is accepted and a 4096 x 4096 weight at 2048
    rows takes the matrix-core input gradient (no split, no workspace) and
    the two-pass GEMM (33 KiB records per 128 x 64 weight tile)."""
    lib = B.load()
    big = _desc(N=65536, K=65536)
    assert big.bytes >= 1 << 32
    out = ctypes.c_size_t(7)
    assert lib.ht_linear_backward_workspace(ctypes.byref(big), 2048, ctypes.byref(out)) == 1
    with pytest.raises(B.HTError):
        B.ht_linear_workspace(big, 2048, B.HT_PATH_GEMM)
    assert lib.ht_linear_backward_workspace(ctypes.byref(_desc(N=32768, K=65536)), 1, ctypes.byref(out)) == 0
    small = _desc(N=4096, K=4096)
    assert lib.ht_linear_backward_workspace(ctypes.byref(small), 2048, ctypes.byref(out)) == 0
    assert out.value == 0
    assert B.ht_linear_workspace(small, 2048, B.HT_PATH_GEMM) == 32 * 64 * 33 * 1024


def test_backward_weight_argument_checks():
    """Argument checks of ht_linear_backward_weight (return before any GPU
    call): 1 EINVAL, 2 ESHAPE, 3 EALIGN."""
    f = B.load().ht_linear_backward_weight
    dy, x, dw = 0x200000, 0x300000, 0x400000
    assert f(dy, 2, 64, x, 128, 64, 128, None, 128, 0, None) == 1            # no dw
    assert f(None, 2, 64, x, 128, 64, 128, dw, 128, 0, None) == 1            # no dy with M > 0
    assert f(dy, -1, 64, x, 128, 64, 128, dw, 128, 0, None) == 2             # M < 0
    assert f(dy, 2, 64, x, 126, 64, 126, dw, 128, 0, None) == 2              # K % 4
    assert f(dy, 2, 63, x, 128, 64, 128, dw, 128, 0, None) == 2              # lddy < N
    assert f(dy, 2, 64, x, 130, 64, 128, dw, 128, 0, None) == 2              # ldx % 4
    assert f(dy, 2, 64, x, 128, 64, 128, dw, 124, 0, None) == 2              # lddw < K
    assert f(dy, 2, 64, x, 128, 4 * 65536, 128, dw, 128, 0, None) == 2       # too many row groups
    assert f(dy, 2, 64, x + 8, 128, 64, 128, dw, 128, 0, None) == 3          # misaligned x


# ---------------------------------------------------------------------------
# Descriptors that do not match their layout, and packed buffers whose block
# index is not that of a format map, are refused on the host.
# ---------------------------------------------------------------------------
def _packed_host(orc, N=37, K=320, R=16, seed=3):
    import numpy as np
    rng = np.random.default_rng(seed)
    W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(N, K // 64)).astype(np.uint8)
    buf = orc.pack(W, fmt, R)
    counts = [int(c) for c in np.bincount(fmt.ravel(), minlength=5)]
    return _desc(N, K, R, counts=counts), buf, fmt


@pytest.mark.parametrize("N,K,R", [(37, 320, 16), (64, 256, 4), (5, 64, 1), (33, 192, 8), (16, 128, 2)])
def test_check_packed_accepts_packer_output(orc, N, K, R):
    import numpy as np
    d, buf, fmt = _packed_host(orc, N, K, R)
    out = np.full_like(fmt, 9)
    B.ht_check_packed(d, buf, out)
    np.testing.assert_array_equal(out, fmt)


def _kbidx(d, buf):
    import numpy as np
    nk = int(d.n_tiles) * (int(d.K) // 64) + 1
    return buf[int(d.off_kbidx):int(d.off_kbidx) + 20 * nk].view(np.uint32).reshape(5, nk)


def _ids(d, buf, f):
    import numpy as np
    return buf[int(d.off_ids[f]):int(d.off_ids[f]) + 2 * int(d.counts[f])].view(np.uint16)


def _t_kbidx_start(d, buf):
    _kbidx(d, buf)[1, 0] = 1


def _t_kbidx_decreasing(d, buf):
    k = _kbidx(d, buf)
    f = int(k[:, -1].argmax())
    c = int((k[f] > 0).argmax())   # first column with a nonzero prefix
    k[f, c] = k[f, c + 1] + 1 if c + 1 < k.shape[1] else k[f, c] + 1


def _t_kbidx_total(d, buf):
    _kbidx(d, buf)[4, -1] += 1


def _t_id_wrong_kb(d, buf):
    ids = _ids(d, buf, 1)
    ids[0] += int(d.row_tile)      # same row, next K-block


def _t_id_row_past_ragged_tile(d, buf):
    # the last tile of N = 37, R = 16 holds rows 0..4: move a block there to row 7
    k = _kbidx(d, buf)
    KB = int(d.K) // 64
    c = (int(d.n_tiles) - 1) * KB
    for f in range(5):
        if k[f, c + 1] > k[f, c]:
            ids = _ids(d, buf, f)
            j = int(k[f, c])
            ids[j] = (int(ids[j]) & 0xFFF0) | 7
            return
    raise AssertionError("no block in the last column")


def _t_duplicate_row(d, buf):
    k = _kbidx(d, buf)
    for f in range(5):
        for c in range(k.shape[1] - 1):
            if k[f, c + 1] - k[f, c] >= 2:
                ids = _ids(d, buf, f)
                ids[int(k[f, c]) + 1] = ids[int(k[f, c])]
                return
    raise AssertionError("no column with two blocks of one format")


def _t_rows_out_of_order(d, buf):
    k = _kbidx(d, buf)
    for f in range(5):
        for c in range(k.shape[1] - 1):
            if k[f, c + 1] - k[f, c] >= 2:
                ids = _ids(d, buf, f)
                j = int(k[f, c])
                ids[j], ids[j + 1] = int(ids[j + 1]), int(ids[j])
                return
    raise AssertionError("no column with two blocks of one format")


def _t_offset(d, buf):
    d.off_payload[4] += 256


def _t_bytes(d, buf):
    d.bytes += 256


def _t_counts_swapped(d, buf):
    # counts that still add up and give a consistent layout, but not the
    # index's totals
    c = [int(v) for v in d.counts]
    c[0], c[4] = c[0] + 1, c[4] - 1
    nd = _with_counts(d, c)
    ctypes.memmove(ctypes.addressof(d), ctypes.addressof(nd), ctypes.sizeof(d))


def _t_version(d, buf):
    d.layout_version = 2


@pytest.mark.parametrize("tamper", [_t_kbidx_start, _t_kbidx_decreasing, _t_kbidx_total, _t_id_wrong_kb,
                                    _t_id_row_past_ragged_tile, _t_duplicate_row, _t_rows_out_of_order,
                                    _t_offset, _t_bytes, _t_counts_swapped, _t_version])
def test_check_packed_refuses_tampering(orc, tamper):
    d, buf, _ = _packed_host(orc)
    tamper(d, buf)
    with pytest.raises(B.HTError) as e:
        B.ht_check_packed(d, buf)
    assert e.value.code == 1


def test_check_packed_short_buffer(orc):
    d, buf, _ = _packed_host(orc)
    with pytest.raises(B.HTError) as e:
        B.ht_check_packed(d, buf[:-1])
    assert e.value.code == 4


@pytest.mark.parametrize("tamper", [_t_offset, _t_bytes, _t_version])
def test_entry_points_refuse_tampered_descriptors(tamper):
    """Every entry point that takes a descriptor refuses one whose offsets or
    size do not match its layout, before anything is launched."""
    lib = B.load()
    d = _desc(N=256, K=512)
    tamper(d, None)
    out = ctypes.c_size_t(0)
    x, y, ws = 0x200000, 0x300000, 0x400000
    assert lib.ht_linear_workspace(ctypes.byref(d), 1, 0, ctypes.byref(out)) == 1
    assert lib.ht_linear_forward(ctypes.byref(d), x, 1, 512, y, 256, 0, 0, ws, 1 << 20, None) == 1
    assert lib.ht_linear_backward_workspace(ctypes.byref(d), 1, ctypes.byref(out)) == 1
    assert lib.ht_linear_backward_data(ctypes.byref(d), y, 1, 256, x, 512, ws, 1 << 20, None) == 1
    arr = (ctypes.POINTER(B.PackedWeight) * 1)(ctypes.pointer(d))
    assert lib.ht_mlp_workspace(arr, 1, 1, ctypes.byref(out)) == 1
    assert lib.ht_mlp_forward(arr, 1, x, 1, 512, y, 256, None, 0, ws, 1 << 20, None) == 1


def test_backward_data_requires_aligned_buffer():
    lib = B.load()
    d = _desc(N=256, K=512, base=0x100008)
    assert lib.ht_linear_backward_data(ctypes.byref(d), 0x200000, 1, 256, 0x300000, 512, 0x400000, 1 << 20,
                                       None) == 3


def test_noalloc_argument_checks():
    """ht_linear_forward_noalloc refuses on the host what ht_linear_forward
    refuses, and a call needing more than its fixed array (32 MiB per GPU)
    with HT_ESMALL, before any HIP call."""
    lib = B.load()
    f = lib.ht_linear_forward_noalloc
    x, y = 0x200000, 0x300000
    d = _desc(N=512, K=14336)
    bad = _desc(N=512, K=14336)
    bad.bytes += 256
    assert f(None, x, 1, 14336, y, 512, 0, 0, None) == 1
    assert f(ctypes.byref(bad), x, 1, 14336, y, 512, 0, 0, None) == 1
    assert f(ctypes.byref(d), x, 0, 14336, y, 512, 0, 0, None) == 2
    assert f(ctypes.byref(d), x, 1, 14336, y, 512, 0, 9, None) == 1
    assert f(ctypes.byref(_desc(R=8)), x, 8, 256, y, 256, 0, B.HT_PATH_GEMV_MFMA, None) == 1
    need = B.ht_linear_workspace(d, 2048, B.HT_PATH_GEMM_I8)      # the encoded x of 2048 x 14336 and more
    assert need > 32 << 20
    assert f(ctypes.byref(d), x, 2048, 14336, y, 512, 0, B.HT_PATH_GEMM_I8, None) == 4


def test_refresh_argument_checks(orc):
    """ht_refresh_bytes bounds every plan's packed size; ht_refresh refuses
    bad arguments and ht_refresh_desc a layout larger than the buffer, all on
    the host before any launch."""
    import itertools
    for (N, K, R) in [(256, 256, 16), (37, 320, 4), (4096, 4096, 16), (5, 64, 1)]:
        bb, wb = B.ht_refresh_bytes(N, K, R)
        assert wb >= 256 + 16 * 2048
        nb = N * (K // 64)
        for f in range(5):   # every single-format plan and a few mixes fit the bound
            c = [0] * 5
            c[f] = nb
            assert orc.pack_layout(N, K, R, c)[0] <= bb
        for c in itertools.product(*[[0, nb // 3] for _ in range(4)]):
            c = list(c) + [nb - sum(c)]
            if c[4] >= 0:
                assert orc.pack_layout(N, K, R, c)[0] <= bb
    with pytest.raises(B.HTError):
        B.ht_refresh_bytes(256, 100, 16)
    lib = B.load()
    f = lib.ht_refresh
    W, fmt, buf, cnt, ws = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    assert f(None, 256, 256, 256, None, 16, fmt, buf, 1 << 20, cnt, ws, 1 << 16, None) == 1
    assert f(W, 256, 256, 128, None, 16, fmt, buf, 1 << 20, cnt, ws, 1 << 16, None) == 2   # ldw < K
    assert f(W, 256, 256, 256, None, 3, fmt, buf, 1 << 20, cnt, ws, 1 << 16, None) == 2    # row tile
    assert f(W, 256, 256, 256, None, 16, fmt, buf + 16, 1 << 20, cnt, ws, 1 << 16, None) == 3  # buf not 256-aligned
    assert f(W, 256, 256, 256, None, 16, fmt, buf, 1 << 20, cnt, ws, 100, None) == 4       # workspace
    p = B.ht_plan_params_default()
    p.eps_int4 = -1.0
    assert f(W, 256, 256, 256, ctypes.byref(p), 16, fmt, buf, 1 << 20, cnt, ws, 1 << 16, None) == 1
    c = [0, 1024, 0, 0, 0]
    size = orc.pack_layout(256, 256, 16, c)[0]
    d = B.ht_refresh_desc(256, 256, 16, c, buf, buf_bytes=size)
    assert int(d.bytes) == size and int(d.base) == buf
    with pytest.raises(B.HTError) as e:
        B.ht_refresh_desc(256, 256, 16, c, buf, buf_bytes=size - 1)
    assert e.value.code == 4
