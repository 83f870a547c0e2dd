"""The fused refresh (ht_refresh: re-plan and re-pack in one pass over W into
buffers allocated in advance) against the oracle: the format map, the
counts and the whole packed buffer byte for byte equal to oracle.plan then
oracle.pack, on the weights the refresh holds in registers and on a larger
one it reads twice."""
import numpy as np
import pytest
import torch

from block_planner_amd import api
from block_planner_amd import binding as B
from block_planner_amd import workloads as wl

pytestmark = pytest.mark.gpu

INT4, INT8, BF16, FP16, FP32 = 0, 1, 2, 3, 4


def dev():
    return torch.device("cuda:0")


def edge_weight(rows=48, per_row=5, seed=3):
    E = wl.edge_blocks(seed)
    rng = np.random.default_rng(seed + 11)
    idx = rng.integers(0, E.shape[0], size=(rows, per_row))
    idx.reshape(-1)[:E.shape[0]] = np.arange(E.shape[0])
    return np.ascontiguousarray(E[idx].reshape(rows, per_row * 64).astype(np.float32))


def t_weight(n, k, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_t(4, size=(n, k)) * 0.02).astype(np.float32)
    W.reshape(-1)[rng.choice(W.size, size=max(1, W.size // 300), replace=False)] *= 30
    return W


def oracle_kw(kw):
    kw = dict(kw)
    force = kw.pop("force_format", -1)
    return dict(kw, force=force)


def check_refresh(orc, W, R, kw, what, st=None):
    Wg = torch.from_numpy(W).to(dev())
    N, K = W.shape
    st = api.refresh_state(N, K, R, dev()) if st is None else st
    pw = api.refresh(Wg, st, **kw)
    torch.cuda.synchronize()
    fmt_or = orc.plan(W, **oracle_kw(kw))
    np.testing.assert_array_equal(st.fmt.cpu().numpy(), fmt_or, err_msg=f"{what}: format map")
    assert pw.counts == [int(c) for c in np.bincount(fmt_or.ravel(), minlength=5)], what
    ref = orc.pack(W, fmt_or, R)
    assert int(pw.desc.bytes) == ref.size, what
    got = pw.buf.cpu().numpy()
    assert np.array_equal(got, ref), f"{what}: {int((got != ref).sum())} bytes differ"
    # the descriptor is the packer's
    d2 = api.pack(Wg, torch.from_numpy(fmt_or).to(dev()), row_tile=R).desc
    for f in ("N", "K", "row_tile", "n_tiles", "off_kbidx", "bytes"):
        assert getattr(pw.desc, f) == getattr(d2, f), (what, f)
    assert list(pw.desc.off_ids) == list(d2.off_ids) and list(pw.desc.off_payload) == list(d2.off_payload)
    assert int(st.ws[8:12].view(torch.int32).item()) == 0
    return st


@pytest.mark.parametrize("name,R,kw", [
    ("small weight", 16, {}),
    ("small weight", 4, {}),
    ("small weight", 1, {}),
    ("ragged", 16, {}),
    ("ragged", 2, {"eps_int4": 0.16}),
    ("edge blocks", 8, {}),
    ("edge blocks", 16, {"prefer_bf16": False}),
    ("edge blocks", 16, {"eps_bf16": 0.004, "eps_fp16": 0.0005, "prefer_bf16": False}),
    ("small weight", 16, {"eps_bf16": 0.01, "eps_fp16": 0.01}),
    ("small weight", 16, {"force_format": INT4}),
    ("edge blocks", 4, {"force_format": INT8}),
    ("small weight", 8, {"force_format": FP16}),
])
def test_refresh_matches_plan_and_pack(orc, name, R, kw):
    W = {"small weight": lambda: wl.small_weight(seed=5),
         "ragged": lambda: t_weight(37, 320, 21),
         "edge blocks": lambda: edge_weight()}[name]()
    check_refresh(orc, W, R, kw, f"{name} R={R} {kw}")


def test_refresh_full_mlp_layer(orc):
    """A 4096 x 4096 layer of the benchmark MLP: held in registers between
    planning and scatter (W read once)."""
    check_refresh(orc, wl.mlp_weight(2), 16, {}, "mlp4096 layer 2")


def test_refresh_large_weight_reads_twice(orc):
    """The Llama-8B-shaped gate projection (14336 x 4096, 235 MB of fp32):
    more than the resident workgroups hold, so W is read again for the
    scatter; the result is the same."""
    shp = [s for s in wl.llama8b_shapes() if s.name == "gate"][0]
    check_refresh(orc, wl.llama8b_weight(0, shp), 16, {}, "llama8b gate")


def test_refresh_twice_on_one_workspace(orc):
    """Consecutive refreshes of a changing weight on the same buffers: each
    call's totals carry its own tag, so none reads the previous call's."""
    st = None
    for step in range(4):
        W = t_weight(300, 1024, 40 + step)
        st = check_refresh(orc, W, 16, {"eps_int4": 0.04 * (step + 1)}, f"step {step}", st)


def test_refresh_buffer_too_small(orc):
    """A buffer smaller than the new layout: map and counts are written, the
    buffer is not, the flag word says so and the descriptor is refused."""
    W = wl.small_weight(seed=6)
    N, K = W.shape
    bb, wb = B.ht_refresh_bytes(N, K, 16)
    c4 = [N * (K // 64), 0, 0, 0, 0]
    small = orc.pack_layout(N, K, 16, c4)[0]         # room for an all-INT4 plan only
    st = api.refresh_state(N, K, 16, dev())
    st.buf = api._aligned_empty(small, dev())
    st.buf.fill_(0xA5)
    B.ht_refresh(torch.from_numpy(W).to(dev()), st.fmt, st.buf, st.counts, st.ws, api.plan_params(), row_tile=16)
    torch.cuda.synchronize()
    assert int(st.ws[12:16].view(torch.int32).item()) == 1
    assert torch.all(st.buf == 0xA5)
    np.testing.assert_array_equal(st.fmt.cpu().numpy(), orc.plan(W))
    with pytest.raises(B.HTError) as e:
        B.ht_refresh_desc(N, K, 16, [int(v) for v in st.counts.cpu()], st.buf)
    assert e.value.code == 4


def test_hyperlinear_refresh_every_trains(orc):
    """HyperLinear(refresh_every=1): every forward after the first re-plans
    and re-packs the updated master with the fused pass; after SGD steps the
    module's map and packed bytes equal the oracle's plan and pack of the
    current master, and its output matches the oracle's linear."""
    from block_planner_amd import nn as htnn

    torch.manual_seed(0)
    lin = htnn.HyperLinear(256, 192, refresh_every=1, device=dev())
    opt = torch.optim.SGD(lin.parameters(), lr=0.05)
    x = torch.randn(8, 256, device=dev())
    for _ in range(3):
        y = lin(x)
        loss = (y * y).sum()
        opt.zero_grad()
        loss.backward()
        opt.step()
    y = lin(x)                                            # refreshes from the updated master
    torch.cuda.synchronize()
    W = lin.weight.detach().cpu().numpy()
    fmt_or = orc.plan(W)
    np.testing.assert_array_equal(lin.fmt.cpu().numpy(), fmt_or)
    assert np.array_equal(lin.packed.buf.cpu().numpy(), orc.pack(W, fmt_or, 16))
    xb = x.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    y_or = orc.linear(W, fmt_or, xb)
    assert np.max(np.abs(y.detach().cpu().numpy() - y_or)) <= 1e-3 * np.max(np.abs(y_or))
