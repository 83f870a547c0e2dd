"""Pins of the CPU oracle against facts that do not come from the oracle itself:
library routines (numpy / torch casts and IEEE fp32 division), exact rational
arithmetic, closed forms and invariants.  None of these tests needs a GPU.

Each test names the plausible oracle mistake it would catch.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from block_planner_amd import workloads as wl

INT4, INT8, BF16, FP16, FP32 = 0, 1, 2, 3, 4


# ---------------------------------------------------------------------------
# Library-routine references (independent of the oracle's C code)
# ---------------------------------------------------------------------------
def np_int_quant(w: np.ndarray, Q: int):
    """numpy fp32: s = fl32(amax / Q), q = clip(rint(fl32(w / s)), -Q, Q)."""
    w = w.astype(np.float32)
    amax = np.max(np.abs(w))
    s = np.float32(amax) / np.float32(Q)
    if s == 0 or not np.isfinite(s):
        return s, np.zeros(64, np.int8)
    with np.errstate(over="ignore", under="ignore"):
        t = (w / s).astype(np.float32)
    q = np.clip(np.rint(t), -Q, Q).astype(np.int8)
    return s, q


def torch_bf16(w: np.ndarray) -> np.ndarray:
    return torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def np_fp16(w: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return w.astype(np.float32).astype(np.float16).astype(np.float64)


def exact_recon(w: np.ndarray, f: int):
    """Reconstruction as exact Fractions, each format from a library routine."""
    if f in (INT4, INT8):
        s, q = np_int_quant(w, 7 if f == INT4 else 127)
        fs = Fraction(float(s))
        return [Fraction(int(v)) * fs for v in q]
    if f == BF16:
        return [Fraction(float(v)) for v in torch_bf16(w)]
    if f == FP16:
        vals = np_fp16(w)
        if not np.all(np.isfinite(vals)):
            return None  # overflow: infinite error
        return [Fraction(float(v)) for v in vals]
    return [Fraction(float(v)) for v in w.astype(np.float32)]


def exact_pick(w: np.ndarray, eps, prefer_bf16=True):
    """First admissible format with err^2 <= eps^2 * nrm^2 evaluated exactly.
    Returns (format, near_tie) where near_tie flags a decision within 1e-9
    relative of the threshold (fp64 rounding could then legitimately differ)."""
    w = w.astype(np.float32)
    if not np.all(np.isfinite(w)):
        return FP32, False
    wf = [Fraction(float(v)) for v in w]
    nrm2 = sum(v * v for v in wf)
    order = [INT4, INT8, BF16, FP16] if prefer_bf16 else [INT4, INT8, FP16, BF16]
    near = False
    for f in order:
        rec = exact_recon(w, f)
        if rec is None:
            continue
        err2 = sum((a - b) * (a - b) for a, b in zip(wf, rec))
        thr = Fraction(float(eps[f])) ** 2 * nrm2
        if thr > 0 and abs(err2 - thr) <= thr * Fraction(1, 10**9):
            near = True
        if err2 <= thr:
            return f, near
    return FP32, near


# ---------------------------------------------------------------------------
# 16-bit rounding: definition vs torch / numpy casts
# ---------------------------------------------------------------------------
def _rounding_probe_values():
    rng = np.random.default_rng(5)
    v = [rng.normal(size=4000).astype(np.float32),
         (rng.normal(size=500) * 1e-39).astype(np.float32),          # fp32 subnormal
         (rng.normal(size=500) * 1e-6).astype(np.float32),           # fp16 subnormal range
         (rng.normal(size=500) * 3e4).astype(np.float32),            # fp16 near max
         (rng.normal(size=200) * 1e38).astype(np.float32),           # bf16 near max
         np.array([0.0, -0.0, 65504, 65519.996, 65520, -65520, 3.3895314e38, 3.4e38,
                   2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -126, 2.0 ** -133,
                   1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11],
                  np.float32)]
    # exact ties for both formats: mantissa bit just below the kept ones set
    base = rng.normal(size=300).astype(np.float32).view(np.uint32)
    v.append(((base & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32))
    v.append(((base & np.uint32(0xFFFFE000)) | np.uint32(0x1000)).view(np.float32))
    return np.concatenate(v).astype(np.float32)


def test_bf16_rounding_matches_torch_cast(orc):
    """Catches a wrong tie rule, a wrong subnormal spacing or a wrong overflow
    threshold in the bfloat16 definition."""
    vals = _rounding_probe_values()
    ref = torch.from_numpy(vals).to(torch.bfloat16)
    ref_bits = ref.view(torch.int16).numpy().view(np.uint16)
    ref_vals = ref.to(torch.float64).numpy()
    for v, rb, rv in zip(vals, ref_bits, ref_vals):
        r = orc.bf16_round(float(v))
        assert (r == rv) or (np.isnan(r) and np.isnan(rv)), (v, r, rv)
        assert np.signbit(r) == np.signbit(rv)
        assert orc.bf16_bits(r) == rb, (v, hex(orc.bf16_bits(r)), hex(rb))


def test_fp16_rounding_matches_numpy_cast(orc):
    """Catches a wrong tie rule, a wrong fp16 subnormal quantum or a wrong
    overflow point (65520 must round to infinity)."""
    vals = _rounding_probe_values()
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16)
    for v, rh in zip(vals, ref):
        r = orc.fp16_round(float(v))
        rv = float(rh)
        assert r == rv, (v, r, rv)
        assert np.signbit(r) == np.signbit(rv)
        assert orc.fp16_bits(r) == int(np.array(rh).view(np.uint16)), v


# ---------------------------------------------------------------------------
# Integer codes and scales: fp32 library arithmetic
# ---------------------------------------------------------------------------
def _quant_probe_blocks():
    rng = np.random.default_rng(11)
    blocks = [rng.normal(size=64) * 0.02, rng.standard_t(4, size=64) * 0.1,
              rng.normal(size=64) * 1e-30, rng.normal(size=64) * 1e30]
    blocks = [b.astype(np.float32) for b in blocks]
    blocks += list(wl.edge_blocks())
    for _ in range(300):
        b = rng.normal(size=64) * 10.0 ** rng.uniform(-20, 20)
        blocks.append(b.astype(np.float32))
    return [b for b in blocks if np.all(np.isfinite(b))]


@pytest.mark.parametrize("Q", [7, 127])
def test_int_codes_match_numpy_fp32(orc, Q):
    """Catches a scale computed in double, a multiply-by-reciprocal instead of
    the fp32 division, round-half-away instead of half-even, or a missing clamp."""
    for b in _quant_probe_blocks():
        s, q = orc.int_quant_block(b, Q)
        s_ref, q_ref = np_int_quant(b, Q)
        assert np.float32(s).view(np.uint32) == np.float32(s_ref).view(np.uint32), b
        np.testing.assert_array_equal(q, q_ref)


def test_subnormal_scale_needs_clamp(orc):
    """amax = 10 * 2^-149 gives s4 = 2^-149 (fp32 subnormal rounding), so w / s
    is 10 and the code must clamp to 7 (the symmetric range)."""
    w = np.zeros(64, np.float32)
    w[0] = np.float32(10 * 2.0 ** -149)
    s, q = orc.int_quant_block(w, 7)
    assert s == np.float32(2.0 ** -149)
    assert q[0] == 7 and np.all(q[1:] == 0)


# ---------------------------------------------------------------------------
# Exact rational brute force of the whole pick
# ---------------------------------------------------------------------------
def _brute_force_blocks():
    rng = np.random.default_rng(1234)
    out = []
    for _ in range(120):
        out.append((rng.normal(size=64) * 0.02).astype(np.float32))
    for _ in range(60):
        out.append((rng.standard_t(3, size=64) * 0.05).astype(np.float32))
    for _ in range(40):
        b = (rng.normal(size=64) * 0.02).astype(np.float32)
        b[rng.integers(64)] = np.float32(rng.normal() * 2)
        out.append(b)
    out += list(wl.edge_blocks())
    for _ in range(30):   # bfloat16-valued with an outlier: BF16 candidates
        b = rng.normal(size=64).astype(np.float32)
        b = (b.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
        b[rng.integers(64)] = np.float32(60.0)
        out.append(b)
    for _ in range(30):   # float16-valued: FP16 candidates
        b = (rng.normal(size=64)).astype(np.float16).astype(np.float32)
        b[rng.integers(64)] = np.float32(100.0)
        out.append(b)
    for _ in range(30):   # INT4-ish: few distinct levels, near-admissible for INT4
        lv = rng.integers(-7, 8, size=64).astype(np.float32)
        b = (lv + rng.normal(size=64) * 0.2).astype(np.float32) * np.float32(0.01)
        out.append(b)
    return out


def test_pick_is_exact_minimum_default_eps(orc):
    """The chosen format equals the first format whose exact squared error is
    within eps^2 * ||w||^2 (rational arithmetic).  Catches a reversed format
    order, a strict '<' instead of '<=', a threshold on the unsquared norm, a
    dropped term in the error sum and a wrong prefer_bf16 tie-break."""
    eps = [0.08, 0.01, 0.0, 0.0]
    checked = 0
    for pref in (True, False):
        for b in _brute_force_blocks():
            want, near = exact_pick(b, eps, pref)
            got = orc.pick_block(b, *eps, prefer_bf16=pref)
            if near:
                continue
            assert got == want, (pref, got, want, b)
            checked += 1
    assert checked > 600


def test_pick_is_exact_near_threshold(orc):
    """Thresholds placed within +-0.5% of each block's own exact relative INT4
    and INT8 error, so the decision is taken right at the boundary."""
    rng = np.random.default_rng(99)
    checked = 0
    for trial in range(150):
        b = (rng.normal(size=64) * 0.03).astype(np.float32)
        wf = [Fraction(float(v)) for v in b]
        nrm2 = sum(v * v for v in wf)
        rel = {}
        for f in (INT4, INT8):
            rec = exact_recon(b, f)
            rel[f] = float(sum((a - c) ** 2 for a, c in zip(wf, rec)) / nrm2) ** 0.5
        target = INT4 if trial % 2 == 0 else INT8
        eps = [0.0, 0.0, 0.0, 0.0]
        eps[INT8] = 0.5 if target == INT4 else rel[INT8] * (1 + rng.uniform(-0.005, 0.005))
        eps[INT4] = rel[INT4] * (1 + rng.uniform(-0.005, 0.005)) if target == INT4 else 0.0
        want, near = exact_pick(b, eps)
        got = orc.pick_block(b, *eps)
        if near:
            continue
        assert got == want, (trial, got, want, eps, rel)
        checked += 1
    assert checked > 100


def test_plan_matches_block_picks_on_tiny_matrices(orc):
    """Whole-matrix planning addresses block (n, kb) as W[n, 64kb:64kb+64]
    (row-major K-blocks); catches a transposed or strided block walk."""
    rng = np.random.default_rng(3)
    for (N, K) in [(1, 64), (2, 128), (3, 192), (8, 256), (5, 320)]:
        W = (rng.normal(size=(N, K)) * 0.02).astype(np.float32)
        W[rng.integers(N), rng.integers(K)] = 3.0
        fmt = orc.plan(W)
        for n in range(N):
            for kb in range(K // 64):
                want, near = exact_pick(W[n, kb * 64:(kb + 1) * 64], [0.08, 0.01, 0.0, 0.0])
                if not near:
                    assert fmt[n, kb] == want


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------
def test_int8_grid_blocks_reconstruct_exactly(orc):
    """w_i = k_i * 2^e with |k_i| <= 127 and max |k_i| = 127: s8 = 2^e exactly,
    q = k, zero error; INT8 is picked unless INT4 already passes."""
    rng = np.random.default_rng(21)
    for e in (-20, -7, 0, 3, 30):
        k = rng.integers(-127, 128, size=64)
        k[rng.integers(64)] = -127 if rng.integers(2) else 127
        w = (k * 2.0 ** e).astype(np.float32)
        s, q = orc.int_quant_block(w, 127)
        assert s == np.float32(2.0 ** e)
        np.testing.assert_array_equal(q, k.astype(np.int8))
        assert orc.block_err2(w, INT8) == 0.0
        assert orc.pick_block(w, eps_int4=0.0) == INT8
        assert orc.pick_block(w, force=INT8) == INT8


def test_int4_grid_blocks_pick_int4_with_zero_error(orc):
    rng = np.random.default_rng(22)
    for e in (-9, 0, 5):
        k = rng.integers(-7, 8, size=64)
        k[0] = 7
        w = (k * 2.0 ** e).astype(np.float32)
        s, q = orc.int_quant_block(w, 7)
        assert s == np.float32(2.0 ** e)
        np.testing.assert_array_equal(q, k.astype(np.int8))
        assert orc.block_err2(w, INT4) == 0.0
        assert orc.pick_block(w, eps_int4=0.0, eps_int8=0.0) == INT4


def test_non_pow2_grid_is_near_exact(orc):
    """A non-power-of-two grid step gives a rounded scale: the INT8 error is
    tiny (relative ~1e-7) but not zero -- a bound, not an equality."""
    k = np.arange(-63, 65) [:64].astype(np.float64)
    k[-1] = 127
    w = (k * 3.0).astype(np.float32)
    rel = (orc.block_err2(w, INT8) / orc.block_nrm2(w)) ** 0.5
    assert rel < 1e-6


def test_fp32_blocks_have_zero_error(orc):
    rng = np.random.default_rng(23)
    for _ in range(20):
        w = (rng.normal(size=64) * 0.02).astype(np.float32)
        assert orc.block_err2(w, FP32) == 0.0
        assert orc.pick_block(w, eps_int4=0.0, eps_int8=0.0) == FP32


def test_zero_block_is_int4_with_zero_scale(orc):
    w = np.zeros(64, np.float32)
    s, q = orc.int_quant_block(w, 7)
    assert s == 0.0 and not q.any()
    assert orc.pick_block(w) == INT4
    w[::3] = -0.0
    assert orc.pick_block(w) == INT4


def test_nonfinite_blocks_are_fp32(orc):
    for b in wl.edge_blocks():
        if not np.all(np.isfinite(b)):
            assert orc.pick_block(b) == FP32


def test_block_norm_matches_exact_sum(orc):
    """nrm2 is the pairwise fp64 sum of exact squares: within 64 ulp of the
    exact rational sum (catches a dropped or duplicated term)."""
    rng = np.random.default_rng(8)
    for _ in range(50):
        w = (rng.normal(size=64) * 10.0 ** rng.uniform(-10, 10)).astype(np.float32)
        exact = sum(Fraction(float(v)) ** 2 for v in w)
        got = orc.block_nrm2(w)
        assert abs(Fraction(got) - exact) <= exact * Fraction(64, 2 ** 52)


def test_pairwise_tree_order(orc):
    """The sums are the balanced pairwise tree in natural order, not a
    left-to-right loop.  One square of 2^40 followed by 63 squares of 2^-14:
    left to right, each 2^-14 is below half an ulp of 2^40 and is absorbed;
    in the tree the small squares first add up among themselves and survive."""
    w = np.full(64, np.float32(2.0 ** -7), np.float32)
    w[0] = np.float32(2.0 ** 20)
    t = [float(v) * float(v) for v in w]

    def tree(a, b):
        if b - a == 1:
            return t[a]
        m = (a + b) // 2
        return tree(a, m) + tree(m, b)

    seq = 0.0
    for v in t:
        seq += v
    assert tree(0, 64) != seq          # the input separates the two orders
    assert orc.block_nrm2(w) == tree(0, 64)
    assert orc.block_err2(w, FP32) == 0.0


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------
def test_sign_symmetry(orc):
    W = wl.small_weight()
    f1 = orc.plan(W)
    f2 = orc.plan(-W)
    np.testing.assert_array_equal(f1, f2)
    for Q in (7, 127):
        s1, q1 = orc.int_quant(W, Q)
        s2, q2 = orc.int_quant(-W, Q)
        np.testing.assert_array_equal(s1, s2)
        np.testing.assert_array_equal(q1, -q2)


def test_int_quant_matrix_layout(orc):
    """The matrix wrapper of the block quantiser: a non-square weight whose
    every block lies on its own power-of-two INT8 grid with a distinct
    exponent, so the scale of block (n, kb) is exactly 2^e[n, kb] and its
    codes are the grid integers (closed form); a transposed or shifted scale
    or code index fails.  Then the wrapper equals the block function block by
    block on edge blocks, at every position of a ragged weight."""
    rng = np.random.default_rng(46)
    N, KB = 7, 5
    e = rng.permutation(N * KB).reshape(N, KB) - 20          # distinct exponents
    k = rng.integers(-127, 128, size=(N, KB, 64))
    k[:, :, 0] = np.where(rng.random((N, KB)) < 0.5, 127, -127)   # |k| reaches 127 in every block
    W = (k * np.ldexp(1.0, e)[:, :, None]).reshape(N, KB * 64).astype(np.float32)
    s, q = orc.int_quant(W, 127)
    np.testing.assert_array_equal(s, np.ldexp(1.0, e).astype(np.float32))
    np.testing.assert_array_equal(q, k.reshape(N, KB * 64).astype(np.int8))
    E = wl.edge_blocks()
    W2 = np.ascontiguousarray(E[rng.integers(0, E.shape[0], size=(9, 3))].reshape(9, 192))
    for Q in (7, 127):
        s2, q2 = orc.int_quant(W2, Q)
        assert s2.shape == (9, 3) and q2.shape == (9, 192)
        for n in range(9):
            for kb in range(3):
                sb, qb = orc.int_quant_block(W2[n, 64 * kb:64 * kb + 64], Q)
                assert s2[n, kb].tobytes() == np.float32(sb).tobytes(), (n, kb)
                np.testing.assert_array_equal(q2[n, 64 * kb:64 * kb + 64], qb)


def test_relu_special_values(orc):
    """The ReLU of the MLP's last layer, by its reading (zero, negative and
    NaN give +0): special values by hand, and max(z, 0) on finite z."""
    z = np.array([2.5, -1.0, 0.0, -0.0, np.nan, -np.nan, np.inf, -np.inf, 5e-324, -5e-324, 1e308])
    r = orc.relu(z)
    want = np.array([2.5, 0.0, 0.0, 0.0, 0.0, 0.0, np.inf, 0.0, 5e-324, 0.0, 1e308])
    assert r.tobytes() == want.tobytes()          # bit patterns: every zero is +0
    zr = np.random.default_rng(47).normal(size=500)
    np.testing.assert_array_equal(orc.relu(zr), np.maximum(zr, 0.0))
    # the hidden layers' ReLU is the same map, then bf16 rounding
    zz = np.concatenate([z, zr])
    assert np.array_equal(orc.relu_bf16(zz), orc.relu_bf16(orc.relu(zz)))
    assert orc.relu_bf16(np.array([np.nan]))[0] == 0


def test_power_of_two_scaling(orc):
    W = wl.small_weight()
    f1 = orc.plan(W)
    s1, q1 = orc.int_quant(W, 127)
    for k in (-6, 5):
        Wk = (W * np.float32(2.0 ** k)).astype(np.float32)
        np.testing.assert_array_equal(orc.plan(Wk), f1)
        sk, qk = orc.int_quant(Wk, 127)
        np.testing.assert_array_equal(qk, q1)
        np.testing.assert_array_equal(sk, (s1 * np.float32(2.0 ** k)).astype(np.float32))


def test_eps_monotonicity(orc):
    """Raising eps never raises a block's format rank; INT4 share grows with
    eps_int4 (the sweep 0.04 <= 0.08 <= 0.16)."""
    W = wl.mlp_weight(0, dim=512)
    plans = [orc.plan(W, eps_int4=e) for e in (0.04, 0.08, 0.16)]
    for a, b in zip(plans, plans[1:]):
        assert np.all(b <= a)
    shares = [np.mean(p == INT4) for p in plans]
    assert shares[0] <= shares[1] <= shares[2]
    p2 = orc.plan(W, eps_int8=0.02)
    assert np.all(p2 <= plans[1])


def test_error_ordering_on_seeded_draws(orc):
    """err_INT4 >= err_INT8 >= err_BF16 >= err_FP32 = 0 on every block of the
    seeded draws (not a theorem; margins are wide on these distributions), and
    err_FP16 <= err_BF16 where every |w| is in fp16's normal range."""
    for W in (wl.small_weight(), wl.mlp_weight(1, dim=256)):
        err2, nrm2 = orc.block_errors(W)
        assert np.all(err2[..., INT4] >= err2[..., INT8])
        assert np.all(err2[..., INT8] >= err2[..., BF16])
        assert np.all(err2[..., BF16] >= err2[..., FP32])
        assert np.all(err2[..., FP32] == 0)
        a = np.abs(W).reshape(W.shape[0], -1, 64)
        normal = np.all((a >= 2.0 ** -14) & (a <= 65504), axis=-1)
        assert np.all(err2[..., FP16][normal] <= err2[..., BF16][normal])


def test_bf16_and_fp16_choice(orc):
    """bfloat16-valued blocks whose outlier defeats INT8 pick BF16 under
    prefer_bf16 and FP16 otherwise (they lie in fp16's normal range, where
    bfloat16 values are fp16-exact); random fp32 blocks never pick either at
    eps = 0."""
    rng = np.random.default_rng(31)
    for _ in range(20):
        # one entry at 1.0, the rest uniform in +-0.05: INT8's half-step error
        # (~0.018 relative) and INT4's zeroing (~0.2) both exceed their eps
        b = rng.uniform(-0.05, 0.05, size=64).astype(np.float32)
        b = (b.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
        b = np.where(np.abs(b) < 2.0 ** -14, np.float32(2.0 ** -5), b).astype(np.float32)
        b[5] = np.float32(1.0)
        assert orc.pick_block(b, eps_bf16=0.5, eps_fp16=0.5) != INT8
        assert orc.pick_block(b, prefer_bf16=True) == BF16
        assert orc.pick_block(b, prefer_bf16=False) == FP16
    for _ in range(20):
        b = rng.normal(size=64).astype(np.float32)
        assert orc.pick_block(b, eps_int4=0.0, eps_int8=0.0) == FP32


# ---------------------------------------------------------------------------
# Linear and MLP
# ---------------------------------------------------------------------------
def test_linear_all_fp32_is_dense_product(orc):
    rng = np.random.default_rng(41)
    W = (rng.normal(size=(48, 256)) * 0.02).astype(np.float32)
    x = wl.to_bf16_bits(rng.normal(size=(3, 256)).astype(np.float32))
    fmt = np.full((48, 4), FP32, np.uint8)
    y = orc.linear(W, fmt, x)
    ref = wl.bf16_bits_to_f32(x).astype(np.float64) @ W.astype(np.float64).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)


def test_linear_int8_grid_is_exact(orc):
    """Power-of-two INT8 grids dequantise exactly, so the linear equals the
    dense product of the original weights."""
    rng = np.random.default_rng(42)
    k = rng.integers(-127, 128, size=(16, 128))
    k[:, 0] = 127
    k[:, 64] = -127
    W = (k * 2.0 ** -9).astype(np.float32)
    fmt = orc.plan(W, eps_int4=0.0)
    assert np.all(fmt == INT8)
    x = wl.to_bf16_bits(rng.normal(size=(2, 128)).astype(np.float32))
    y = orc.linear(W, fmt, x)
    ref = wl.bf16_bits_to_f32(x).astype(np.float64) @ W.astype(np.float64).T
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_linear_uses_dequantised_weights(orc):
    """y equals x_hat . W_hat^T with W_hat from independent library-routine
    reconstructions (numpy fp32 codes, torch bfloat16, numpy float16)."""
    W = wl.small_weight()
    rng = np.random.default_rng(43)
    fmt = rng.integers(0, 5, size=(256, 4)).astype(np.uint8)
    x = wl.to_bf16_bits(wl.small_activation(m=2))
    What = np.zeros((256, 256))
    for n in range(256):
        for kb in range(4):
            blk = W[n, kb * 64:(kb + 1) * 64]
            f = int(fmt[n, kb])
            if f in (INT4, INT8):
                s, q = np_int_quant(blk, 7 if f == INT4 else 127)
                What[n, kb * 64:(kb + 1) * 64] = q.astype(np.float64) * float(s)
            elif f == BF16:
                What[n, kb * 64:(kb + 1) * 64] = torch_bf16(blk)
            elif f == FP16:
                What[n, kb * 64:(kb + 1) * 64] = np_fp16(blk)
            else:
                What[n, kb * 64:(kb + 1) * 64] = blk
    np.testing.assert_array_equal(orc.dequant(W, fmt), What)
    y = orc.linear(W, fmt, x)
    ref = wl.bf16_bits_to_f32(x).astype(np.float64) @ What.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    ys = orc.linear_sampled(W, fmt, x, [0, 1, 1], [0, 17, 255])
    np.testing.assert_array_equal(ys, [y[0, 0], y[1, 17], y[1, 255]])


def test_relu_bf16_matches_torch(orc):
    rng = np.random.default_rng(44)
    z = rng.normal(size=1000) * 3
    h = orc.relu_bf16(z)
    ref = torch.from_numpy(np.maximum(z, 0)).to(torch.bfloat16).view(torch.int16).numpy()
    # fp64 -> bf16 directly equals fp64 -> fp32 -> bf16 except on double-rounding
    # ties, which random normals do not hit
    np.testing.assert_array_equal(h, ref.view(np.uint16))


def test_mlp_composes_layers(orc):
    rng = np.random.default_rng(45)
    Ws = [(rng.normal(size=(128, 128)) * 0.1).astype(np.float32) for _ in range(3)]
    fmts = [orc.plan(W) for W in Ws]
    x = wl.to_bf16_bits(rng.normal(size=(2, 128)).astype(np.float32))
    y, hs = orc.mlp(Ws, fmts, x)
    h = x
    for li, (W, f) in enumerate(zip(Ws, fmts)):
        z = wl.bf16_bits_to_f32(h).astype(np.float64) @ orc.dequant(W, f).T
        if li < 2:
            h = torch.from_numpy(np.maximum(z, 0)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            np.testing.assert_array_equal(h, hs[li])
        else:
            np.testing.assert_allclose(y, np.maximum(z, 0), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Two-plane int8 encoding of x (int8 matrix-core path)
# ---------------------------------------------------------------------------
def _bf16_row(vals):
    return wl.to_bf16_bits(np.array([float(v) for v in vals], np.float32))


def test_x_planes_golden_rows():
    """Hand-worked rows (tests/golden/x_planes.json): catches a wrong exponent
    (off by one at powers of two), a wrong rounding mode (the ties), a hi/lo
    split that truncates instead of flooring (negative entries) and the
    all-zero / non-finite / subnormal special cases."""
    import json
    import os
    import oracle

    data = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "x_planes.json")))
    for row in data["rows"]:
        xb = _bf16_row(row["x"])[None, :]
        assert np.array_equal(wl.bf16_bits_to_f32(xb[0]).astype(np.float64),
                              np.array([float(v) for v in row["x"]])), row["name"]   # inputs are exact bf16
        hi, lo, se = oracle.x_planes(xb)
        assert hi[0].tolist() == row["hi"], row["name"]
        assert lo[0].tolist() == row["lo"], row["name"]
        assert int(se[0]) == row["sexp"], row["name"]


def test_x_planes_properties_random():
    """Properties that fix the encoding on random rows over a wide range of
    magnitudes: the exponent brackets amax (2^(E-1) <= amax < 2^E), v is the
    nearest integer to x * 2^(14-E) with ties to even (checked in exact
    rational arithmetic on a sample), the planes stay in range and combine to
    v, and every entry with |x| >= 2^(E-7) is reproduced exactly."""
    import oracle

    rng = np.random.default_rng(5)
    rows = []
    for scale in (1e-38, 3e-20, 1e-3, 1.0, 7.0, 1e5, 1e30):
        rows.append(rng.standard_t(3, size=192) * scale)
    X = wl.to_bf16_bits(np.array(rows, np.float32))
    hi, lo, se = oracle.x_planes(X)
    xf = wl.bf16_bits_to_f32(X).astype(np.float64)
    assert hi.min() >= -64 and hi.max() <= 64 and lo.min() >= -128 and lo.max() <= 127
    v = 256 * hi.astype(np.int64) + lo.astype(np.int64)
    for m in range(X.shape[0]):
        amax = np.max(np.abs(xf[m]))
        E = int(se[m]) + 14
        assert 2.0 ** (E - 1) <= amax < 2.0 ** E
        xh = np.ldexp(v[m].astype(np.float64), int(se[m]))
        assert np.all(np.abs(xh - xf[m]) <= np.ldexp(0.5, int(se[m])))
        big = np.abs(xf[m]) >= 2.0 ** (E - 7)
        assert np.array_equal(xh[big], xf[m][big])
        for k in range(0, 192, 7):   # exact nearest-even check
            t = Fraction(float(xf[m, k])) * Fraction(2) ** (14 - E)
            fl = t.numerator // t.denominator
            d = t - fl
            want = fl + 1 if d > Fraction(1, 2) or (d == Fraction(1, 2) and fl % 2) else fl
            assert int(v[m, k]) == want, (m, k)



def test_x_planes_scale_and_sign_symmetry():
    """x * 2^j keeps v and moves the exponent by j; -x negates v (round half
    even is symmetric).  Catches an encoding that depends on more than the
    row's exponent, or a floor where a round belongs."""
    import oracle

    rng = np.random.default_rng(6)
    x = rng.normal(size=(3, 128)).astype(np.float32)
    X = wl.to_bf16_bits(x)
    base = wl.bf16_bits_to_f32(X)
    hi, lo, se = oracle.x_planes(X)
    v = 256 * hi.astype(np.int64) + lo
    for j in (-20, -1, 3, 40):
        h2, l2, s2 = oracle.x_planes(wl.to_bf16_bits(base * np.float32(2.0 ** j)))
        assert np.array_equal(256 * h2.astype(np.int64) + l2, v)
        assert np.array_equal(s2, se + j)
    h3, l3, s3 = oracle.x_planes(wl.to_bf16_bits(-base))
    assert np.array_equal(256 * h3.astype(np.int64) + l3, -v)
    assert np.array_equal(s3, se)


def test_linear_xplanes_exact_and_bounded():
    """x_hat . W_hat^T equals the exact linear when every x is representable
    (all |x| >= 2^(E-7)), and otherwise differs by at most
    2^(sexp-1) * sum_k |w_hat[n, k]| per output.  Catches a transposed or
    mis-scaled x_hat in the oracle of the int8 path."""
    import oracle

    rng = np.random.default_rng(7)
    W = (rng.normal(size=(48, 256)) * 0.02).astype(np.float32)
    fmt = oracle.plan(W)
    # representable: entries in {+-1, +-1.5, +-2, ..., +-4}: |x| >= 1 >= 2^(E-7) with E = 3
    xr = rng.choice(np.array([-4, -3, -2, -1.5, -1, 1, 1.5, 2, 3, 4], np.float32), size=(5, 256))
    Xr = wl.to_bf16_bits(xr)
    assert np.allclose(oracle.linear_xplanes(W, fmt, Xr), oracle.linear(W, fmt, Xr), rtol=1e-13, atol=1e-13)
    X = wl.to_bf16_bits(rng.normal(size=(6, 256)).astype(np.float32) * np.float32(3.0))
    yx = oracle.linear_xplanes(W, fmt, X)
    y = oracle.linear(W, fmt, X)
    _, _, se = oracle.x_planes(X)
    bound = np.ldexp(0.5, se)[:, None] * np.abs(oracle.dequant(W, fmt)).sum(axis=1)[None, :]
    assert np.all(np.abs(yx - y) <= bound * (1 + 1e-12))
    assert np.max(np.abs(yx - y)) > 0          # the encoding is not the identity here
    Xn = X.copy()
    Xn[2, 5] = 0x7F80                          # +Inf in row 2
    yn = oracle.linear_xplanes(W, fmt, Xn)
    assert np.all(np.isnan(yn[2])) and np.all(np.isfinite(np.delete(yn, 2, axis=0)))


# ---------------------------------------------------------------------------
# W8A8 encoding of x (one int8 code per entry, one power-of-two scale per
# token and 64-wide K-block)
# ---------------------------------------------------------------------------
def test_x_w8a8_golden_blocks():
    """Hand-worked blocks (tests/golden/x_w8a8.json) laid out as two tokens of
    four K-blocks: catches an exponent off by one at powers of two, a wrong
    rounding mode (ties), a missing clamp (127.5 rounds to 128), a scale per
    token instead of per block, and the zero / non-finite / subnormal cases."""
    import json
    import os
    import oracle

    data = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "x_w8a8.json")))
    blocks = data["blocks"]
    assert len(blocks) == 8
    X = np.zeros((2, 4 * 64), np.uint16)
    for b, blk in enumerate(blocks):
        m, kb = b // 4, b % 4
        for i, bits in blk["x"]:
            X[m, 64 * kb + i] = int(bits, 16)
    q, bexp = oracle.x_w8a8(X)
    for b, blk in enumerate(blocks):
        m, kb = b // 4, b % 4
        want = np.zeros(64, np.int64)
        for i, v in blk["q"]:
            want[i] = v
        assert q[m, 64 * kb:64 * kb + 64].astype(np.int64).tolist() == want.tolist(), blk["what"]
        assert int(bexp[m, kb]) == blk["bexp"], blk["what"]


def test_x_w8a8_properties_random():
    """Random blocks over a wide range of magnitudes, each block of a token
    with its own magnitude: the block exponent brackets the block maximum
    (2^(bexp+6) <= amax < 2^(bexp+7)), every code is the nearest integer to
    x * 2^-bexp with ties to even (exact rational arithmetic on a sample)
    clamped to +-127, and |x - x_hat| <= 2^bexp (half a step, or the clamp)."""
    import oracle

    rng = np.random.default_rng(8)
    scales = np.array([1e-38, 3e-20, 1e-3, 1.0, 7.0, 1e5, 1e30, 2.0 ** -130])
    x = rng.standard_t(3, size=(4, 8 * 64)) * np.repeat(scales[None, :], 64, axis=1)
    X = wl.to_bf16_bits(x.astype(np.float32))
    q, bexp = oracle.x_w8a8(X)
    xf = wl.bf16_bits_to_f32(X).astype(np.float64)
    assert q.min() >= -127 and q.max() <= 127
    xh = oracle.x_hat_w8a8(q, bexp)
    for m in range(4):
        for kb in range(8):
            blk = xf[m, 64 * kb:64 * kb + 64]
            amax, e = np.max(np.abs(blk)), int(bexp[m, kb])
            assert 2.0 ** (e + 6) <= amax < 2.0 ** (e + 7), (m, kb)
            assert np.all(np.abs(xh[m, 64 * kb:64 * kb + 64] - blk) <= np.ldexp(1.0, e))
            for i in range(0, 64, 9):
                t = Fraction(float(blk[i])) * Fraction(2) ** (-e)
                fl = t.numerator // t.denominator
                d = t - fl
                want = fl + 1 if d > Fraction(1, 2) or (d == Fraction(1, 2) and fl % 2) else fl
                want = max(-127, min(127, want))
                assert int(q[m, 64 * kb + i]) == want, (m, kb, i)


def test_x_w8a8_scale_sign_and_block_independence():
    """x * 2^j keeps the codes and moves every block exponent by j; -x negates
    the codes; changing one block leaves every other block's codes and
    exponent unchanged (a per-token scale would not)."""
    import oracle

    rng = np.random.default_rng(9)
    base = wl.bf16_bits_to_f32(wl.to_bf16_bits(rng.normal(size=(3, 256)).astype(np.float32)))
    q, bexp = oracle.x_w8a8(wl.to_bf16_bits(base))
    for j in (-20, -1, 3, 40):
        q2, b2 = oracle.x_w8a8(wl.to_bf16_bits(base * np.float32(2.0 ** j)))
        assert np.array_equal(q2, q) and np.array_equal(b2, bexp + j)
    q3, b3 = oracle.x_w8a8(wl.to_bf16_bits(-base))
    assert np.array_equal(q3, -q) and np.array_equal(b3, bexp)
    big = base.copy()
    big[1, 70] = 1000.0                         # token 1, K-block 1
    q4, b4 = oracle.x_w8a8(wl.to_bf16_bits(big))
    same = np.ones((3, 4), bool)
    same[1, 1] = False
    assert np.array_equal(b4[same], bexp[same]) and b4[1, 1] > bexp[1, 1]
    for m in range(3):
        for kb in range(4):
            if same[m, kb]:
                assert np.array_equal(q4[m, 64 * kb:64 * kb + 64], q[m, 64 * kb:64 * kb + 64])


def test_linear_w8a8_exact_on_grid_and_bounded():
    """x_hat . W_hat^T equals the exact linear when every x is on its block's
    grid, and otherwise differs by at most sum_k 2^bexp[m, k/64] |w_hat[n, k]|;
    a block holding Inf makes its token's outputs NaN."""
    import oracle

    rng = np.random.default_rng(10)
    W = (rng.normal(size=(40, 256)) * 0.02).astype(np.float32)
    fmt = oracle.plan(W)
    # on the grid: every block's max is 4 (E = 3, step 2^-4) and entries are multiples of 1/16
    xr = rng.integers(-64, 65, size=(5, 256)).astype(np.float32) / np.float32(16.0)
    xr[:, ::64] = 4.0
    Xr = wl.to_bf16_bits(xr)
    assert np.allclose(oracle.linear_w8a8(W, fmt, Xr), oracle.linear(W, fmt, Xr), rtol=1e-13, atol=1e-13)
    X = wl.to_bf16_bits(rng.normal(size=(6, 256)).astype(np.float32) * np.float32(3.0))
    yw = oracle.linear_w8a8(W, fmt, X)
    y = oracle.linear(W, fmt, X)
    _, bexp = oracle.x_w8a8(X)
    step = np.repeat(np.ldexp(1.0, bexp), 64, axis=1)
    bound = step @ np.abs(oracle.dequant(W, fmt)).T
    assert np.all(np.abs(yw - y) <= bound * (1 + 1e-12))
    assert np.max(np.abs(yw - y)) > 0
    Xn = X.copy()
    Xn[4, 200] = 0x7F80
    yn = oracle.linear_w8a8(W, fmt, Xn)
    assert np.all(np.isnan(yn[4])) and np.all(np.isfinite(np.delete(yn, 4, axis=0)))


# ---------------------------------------------------------------------------
# Input gradient of the linear (training backward)
# ---------------------------------------------------------------------------
def test_backward_data_is_the_adjoint():
    """<dX, x> = <dY, W_hat x> for every x and dY, with W_hat x taken from the
    oracle's forward (its own C dot products): catches a transposed or
    mis-indexed backward."""
    import oracle

    rng = np.random.default_rng(60)
    W = (rng.standard_t(4, size=(80, 320)) * 0.02).astype(np.float32)
    fmt = rng.integers(0, 5, size=(80, 5)).astype(np.uint8)
    xb = wl.to_bf16_bits(rng.normal(size=(3, 320)).astype(np.float32))
    dy = rng.normal(size=(3, 80)).astype(np.float32)
    dx = oracle.linear_backward_data(W, fmt, dy)
    y = oracle.linear(W, fmt, xb)
    x = wl.bf16_bits_to_f32(xb).astype(np.float64)
    for m in range(3):
        lhs = float(dx[m] @ x[m])
        rhs = float(dy[m].astype(np.float64) @ y[m])
        assert abs(lhs - rhs) <= 1e-12 * (np.abs(dx[m]) @ np.abs(x[m]) + 1e-300)


def test_backward_data_dense_and_grid_cases():
    """All-FP32 blocks: dX = dY W exactly as a dense product of the fp32
    weight; INT8-grid blocks (w = integer * 2^-10): the same, since those
    blocks reconstruct exactly."""
    import oracle

    rng = np.random.default_rng(61)
    W = (rng.normal(size=(48, 192)) * 0.1).astype(np.float32)
    dy = rng.normal(size=(2, 48)).astype(np.float32)
    fmt = np.full((48, 3), FP32, np.uint8)
    np.testing.assert_allclose(oracle.linear_backward_data(W, fmt, dy),
                               dy.astype(np.float64) @ W.astype(np.float64), rtol=1e-13, atol=1e-13)
    G = rng.integers(-127, 128, size=(48, 192)).astype(np.float32)
    G[:, ::64] = 127.0                                   # every block reaches the full range
    Wg = G * np.float32(2.0 ** -10)
    fmt8 = np.full((48, 3), INT8, np.uint8)
    np.testing.assert_allclose(oracle.linear_backward_data(Wg, fmt8, dy),
                               dy.astype(np.float64) @ Wg.astype(np.float64), rtol=1e-13, atol=1e-13)


def test_backward_weight_is_the_adjoint():
    """<dW, V> = <dY, x V^T> for random V, with x V^T from the oracle's
    forward over all-FP32 blocks of V (its own C dot products, exact for
    fp32 V): catches a transposed or mis-indexed weight gradient."""
    import oracle

    rng = np.random.default_rng(62)
    M, N, K = 5, 48, 192
    xb = wl.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    dy = rng.normal(size=(M, N)).astype(np.float32)
    dw = oracle.linear_backward_weight(dy, xb)
    assert dw.shape == (N, K)
    for _ in range(3):
        V = rng.normal(size=(N, K)).astype(np.float32)
        xv = oracle.linear(V, np.full((N, K // 64), FP32, np.uint8), xb)
        lhs = float(np.sum(dw * V.astype(np.float64)))
        rhs = float(np.sum(dy.astype(np.float64) * xv))
        assert abs(lhs - rhs) <= 1e-12 * np.sum(np.abs(dw * V.astype(np.float64)))


def test_backward_weight_brute_force():
    """Tiny case by plain loops, decoding bf16 bits with struct."""
    import struct

    import oracle

    rng = np.random.default_rng(63)
    M, N, K = 3, 4, 5
    xb = rng.integers(0, 1 << 16, size=(M, K)).astype(np.uint16)
    xb[(xb & 0x7F80) == 0x7F80] = 0x3F80            # no Inf / NaN
    dy = rng.normal(size=(M, N)).astype(np.float32)
    f = lambda b: struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]
    dw = oracle.linear_backward_weight(dy, xb)
    for n in range(N):
        for k in range(K):
            ref = 0.0
            for m in range(M):
                ref += float(dy[m, n]) * f(xb[m, k])
            assert dw[n, k] == pytest.approx(ref, rel=1e-12, abs=1e-300)
