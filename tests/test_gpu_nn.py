"""The PyTorch layer (block_planner_amd.nn) on the GPU: scan_model and
wrap_model_with_hypertensor on a small BenchmarkMLP-shaped model, against the
oracle and against ht_mlp_forward's per-layer path; skipped layers;
inference-only memory; refresh; save / load round trip; the input gradient
through HyperLinear."""
import numpy as np
import pytest
import torch

from block_planner_amd import api
from block_planner_amd import binding as B
from block_planner_amd import nn as htnn
from block_planner_amd import workloads as wl

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def mlp_model(dim=256, depth=3, seed=0):
    torch.manual_seed(seed)
    layers = []
    for li in range(depth):
        lin = torch.nn.Linear(dim, dim, bias=False)
        with torch.no_grad():
            lin.weight.copy_(torch.from_numpy(wl.mlp_weight(li, dim=dim, seed=seed)))
        layers += [lin, torch.nn.ReLU()]
    return torch.nn.Sequential(*layers).to(dev())


def test_wrap_matches_oracle_and_library_mlp(orc):
    """Wrapped BenchmarkMLP-shaped model == ht_mlp_forward's per-layer path
    bitwise (same kernels, same bf16 rounding between layers), and each layer
    within the bar of the oracle fed the same bf16 activations."""
    model = mlp_model()
    Ws = [m.weight.detach().cpu().numpy() for m in model if isinstance(m, torch.nn.Linear)]
    plan = htnn.scan_model(model, eps_fp16=0.0, eps_bf16=0.0, prefer_bf16=True)
    assert sorted(plan["layers"]) == ["0", "2", "4"] and not plan["skipped"]
    fmts = [plan["layers"][k]["fmt"].cpu().numpy() for k in ("0", "2", "4")]
    for W, f in zip(Ws, fmts):
        np.testing.assert_array_equal(f, orc.plan(W))
    htnn.wrap_model_with_hypertensor(model, plan, inference_only=True)
    assert all(isinstance(model[i], htnn.HyperLinear) for i in (0, 2, 4))
    x = torch.from_numpy(wl.mlp_activation(5, dim=256)).to(dev())
    with torch.no_grad():
        y = model(x)
    torch.cuda.synchronize()
    # the library's MLP over the same packed layers (each layer on the path AUTO picks)
    xb = x.to(torch.bfloat16)
    y_lib = api.mlp([model[i].packed for i in (0, 2, 4)], xb, path=B.HT_PATH_AUTO)   # 5 rows: per-layer launches
    torch.cuda.synchronize()
    assert torch.equal(y, y_lib)
    # teacher-forced per layer against the oracle
    h = wl.to_bf16_bits(x.cpu().numpy())
    for li, (W, f) in enumerate(zip(Ws, fmts)):
        z = orc.linear(W, f, h)
        with torch.no_grad():
            zg = model[2 * li](torch.from_numpy(wl.bf16_bits_to_f32(h)).to(dev())).cpu().numpy()
        assert np.max(np.abs(zg - z)) <= 1e-3 * np.max(np.abs(z)), li
        h = orc.relu_bf16(z)


def test_skipped_layers_and_options():
    model = torch.nn.Sequential(torch.nn.Linear(128, 64, bias=True), torch.nn.Linear(64, 96, bias=False),
                                torch.nn.Linear(96, 32, bias=False)).to(dev())
    plan = htnn.scan_model(model)
    assert plan["skipped"] == {"0": "has a bias", "2": "in_features is not a multiple of 64"}
    assert list(plan["layers"]) == ["1"]
    with pytest.raises(ValueError):
        htnn.wrap_model_with_hypertensor(model, plan, option="BEST")
    htnn.wrap_model_with_hypertensor(model, plan)
    assert isinstance(model[0], torch.nn.Linear) and isinstance(model[1], htnn.HyperLinear)
    assert isinstance(model[2], torch.nn.Linear)
    with torch.no_grad():
        y = model(torch.randn(3, 128, device=dev()))
    assert y.shape == (3, 32) and torch.all(torch.isfinite(y))


def test_inference_only_memory_and_shapes(orc):
    lin = torch.nn.Linear(512, 320, bias=False).to(dev())
    m = htnn.HyperLinear.from_linear(lin, inference_only=True)
    mem = m.memory_bytes()
    assert mem["master_fp32"] == 0 and mem["packed"] == m.packed.nbytes > 0
    assert mem["packed"] < 512 * 320 * 4                      # smaller than the fp32 master
    keep = htnn.HyperLinear.from_linear(lin, inference_only=False)
    assert keep.memory_bytes()["master_fp32"] == 512 * 320 * 4
    # leading dimensions are kept; an empty batch gives an empty output
    x = torch.randn(2, 3, 512, device=dev())
    with torch.no_grad():
        y = m(x)
        assert y.shape == (2, 3, 320) and y.dtype == torch.float32
        assert m(torch.empty(0, 512, device=dev())).shape == (0, 320)
    W = lin.weight.detach().cpu().numpy()
    xb = wl.to_bf16_bits(x.reshape(6, 512).cpu().numpy())
    yo = orc.linear(W, orc.plan(W), xb)
    assert np.max(np.abs(y.reshape(6, 320).cpu().numpy() - yo)) <= 1e-3 * np.max(np.abs(yo))


def test_refresh_every_replans(orc):
    """With a master weight and refresh_every = 2, the layer re-plans and
    re-packs every second call: after the weight changes, the third call
    uses the new weight."""
    m = htnn.HyperLinear(256, 128, refresh_every=2, device=dev())
    x = torch.randn(4, 256, device=dev())
    with torch.no_grad():
        m(x)
        m(x)
        m.weight.mul_(-2.0)
        y = m(x)
    W = m.weight.detach().cpu().numpy()
    xb = wl.to_bf16_bits(x.cpu().numpy())
    yo = orc.linear(W, orc.plan(W), xb)
    assert np.max(np.abs(y.cpu().numpy() - yo)) <= 1e-3 * np.max(np.abs(yo))


def test_save_load_round_trip(tmp_path):
    model = mlp_model(dim=192, depth=2, seed=3)
    htnn.wrap_model_with_hypertensor(model, htnn.scan_model(model))
    x = torch.randn(7, 192, device=dev())
    with torch.no_grad():
        y = model(x)
    path = str(tmp_path / "m.safetensors")
    htnn.save_hypertensor(model, path)
    fresh = mlp_model(dim=192, depth=2, seed=9)                # other weights: replaced by the load
    htnn.load_hypertensor(fresh, path)
    assert all(isinstance(fresh[i], htnn.HyperLinear) for i in (0, 2))
    assert all(torch.equal(fresh[i].fmt, model[i].fmt) for i in (0, 2))
    with torch.no_grad():
        y2 = fresh(x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("N,K,lead", [(320, 512, (6,)), (200, 192, (2, 3))])
def test_input_gradient_through_hyperlinear(orc, N, K, lead):
    """x.grad after backward through a HyperLinear equals dY . W_hat of the
    oracle (fp64) within the bar; the weight gets no gradient."""
    lin = torch.nn.Linear(K, N, bias=False).to(dev())
    m = htnn.HyperLinear.from_linear(lin, inference_only=False)
    x = torch.randn(*lead, K, device=dev(), requires_grad=True)
    y = m(x)
    g = torch.randn(*lead, N, device=dev())
    (y * g).sum().backward()
    assert x.grad is not None and x.grad.shape == x.shape and m.weight.grad is not None
    W = lin.weight.detach().cpu().numpy()
    g2 = g.reshape(-1, N).cpu().numpy()
    ref = orc.linear_backward_data(W, m.fmt.cpu().numpy(), g2)
    got = x.grad.reshape(-1, K).cpu().numpy()
    assert np.max(np.abs(got - ref)) <= 1e-3 * np.max(np.abs(ref))
    # STE gradient of the master: dY^T . bf16(x)
    xb = wl.to_bf16_bits(x.detach().reshape(-1, K).cpu().numpy())
    refw = orc.linear_backward_weight(g2, xb)
    assert np.max(np.abs(m.weight.grad.cpu().numpy() - refw)) <= 1e-3 * np.max(np.abs(refw))
    # the forward under autograd is the same as without it
    with torch.no_grad():
        assert torch.equal(m(x), y.detach())
    # an optimizer step on the master, then a re-pack: the forward follows the new weight
    torch.optim.SGD([m.weight], lr=0.5).step()
    m.pack()
    with torch.no_grad():
        y2 = m(x).reshape(-1, N).cpu().numpy()
    W2 = m.weight.detach().cpu().numpy()
    assert not np.array_equal(W2, W)
    yo = orc.linear(W2, orc.plan(W2), xb)
    assert np.max(np.abs(y2 - yo)) <= 1e-3 * np.max(np.abs(yo))


def test_inference_only_module_takes_no_weight_gradient():
    lin = torch.nn.Linear(128, 64, bias=False).to(dev())
    m = htnn.HyperLinear.from_linear(lin, inference_only=True)
    x = torch.randn(3, 128, device=dev(), requires_grad=True)
    m(x).sum().backward()
    assert m.weight is None and x.grad is not None and torch.all(torch.isfinite(x.grad))
