"""Argument handling of the PyTorch layer that needs no GPU."""
import pytest
import torch

from block_planner_amd import nn as htnn


def test_options_and_shape_checks():
    model = torch.nn.Sequential(torch.nn.Linear(128, 64, bias=False))
    with pytest.raises(ValueError):
        htnn.wrap_model_with_hypertensor(model, {"layers": {}}, option="BEST")   # undefined planner mode
    assert htnn.wrap_model_with_hypertensor(model, {"layers": {}}, option="PER_BLOCK") is model
    with pytest.raises(KeyError):
        htnn.wrap_model_with_hypertensor(model, {"layers": {"nope": {"fmt": None}}})
    with pytest.raises(ValueError):
        htnn.HyperLinear(128, 64, bias=True)
    with pytest.raises(ValueError):
        htnn.HyperLinear(100, 64)


def test_scan_skips_what_it_cannot_convert():
    model = torch.nn.Sequential(torch.nn.Linear(128, 64, bias=True), torch.nn.Linear(64, 96, bias=False),
                                torch.nn.Linear(96, 32, bias=False))
    plan = htnn.scan_model(model)                 # a CPU model: nothing is planned, nothing runs
    assert plan["layers"] == {}
    assert plan["skipped"] == {"0": "has a bias", "1": "weight is not on a GPU",
                               "2": "in_features is not a multiple of 64"}


def test_trainable_layer_needs_row_tile_16():
    """The backward kernels read 16-row tiles: a trainable module with another
    row tile is refused when it is built, not in its first backward pass."""
    with pytest.raises(ValueError):
        htnn.HyperLinear(128, 64, row_tile=8)
    with pytest.raises(ValueError):
        htnn.HyperLinear(128, 64, row_tile=3, inference_only=True)
    with pytest.raises(ValueError):
        htnn.HyperLinear.from_linear(torch.nn.Linear(128, 64, bias=False), inference_only=False, row_tile=4)


def _write_packed_file(path, orc, tamper=None, fmt_tamper=False):
    """A file in save_hypertensor's format holding one layer packed by the
    oracle's packer (no GPU), optionally tampered with."""
    import json

    import numpy as np
    from safetensors.torch import save_file

    rng = np.random.default_rng(12)
    N, K, R = 37, 320, 16
    W = (rng.normal(size=(N, K)) * 0.05).astype(np.float32)
    fmt = rng.integers(0, 5, size=(N, K // 64)).astype(np.uint8)
    buf = orc.pack(W, fmt, R)
    counts = [int(c) for c in np.bincount(fmt.ravel(), minlength=5)]
    size, offs = orc.pack_layout(N, K, R, counts)
    meta = {"N": N, "K": K, "row_tile": R, "n_tiles": (N + R - 1) // R, "off_kbidx": offs[0], "bytes": size,
            "layout_version": 1, "counts": counts, "off_ids": offs[1:6], "off_scale": offs[6:8],
            "off_payload": offs[8:13]}
    if tamper:
        tamper(meta, buf)
    f = fmt.copy()
    if fmt_tamper:
        f[0, 0] = (f[0, 0] + 1) % 5
    save_file({"lin.packed": torch.from_numpy(buf), "lin.fmt": torch.from_numpy(f)}, path,
              metadata={"hypertensor_layers": json.dumps({"lin": meta})})
    return fmt


def test_read_hypertensor_accepts_a_valid_file(tmp_path, orc):
    import numpy as np
    p = str(tmp_path / "ok.safetensors")
    fmt = _write_packed_file(p, orc)
    [(name, host, d, counts, f)] = htnn.read_hypertensor(p)
    assert name == "lin" and host.numel() == int(d.bytes)
    np.testing.assert_array_equal(f.numpy(), fmt)


def _kb_first(meta, buf):
    buf[meta["off_kbidx"]:meta["off_kbidx"] + 4] = 255


def _id_kb(meta, buf):
    o = meta["off_ids"][1]
    buf[o + 1] ^= 0x10      # id += 16 * 256: a K-block past the weight


@pytest.mark.parametrize("tamper,fmt_tamper", [
    (lambda m, b: m.__setitem__("off_kbidx", 256), False),             # offsets not the layout's
    (lambda m, b: m.__setitem__("bytes", m["bytes"] + 256), False),    # size not the buffer's
    (lambda m, b: m["counts"].__setitem__(0, m["counts"][0] + 1), False),
    (lambda m, b: m.__setitem__("off_ids", m["off_ids"][:4]), False),  # malformed field
    (_kb_first, False),                                                # index does not start at 0
    (_id_kb, False),                                                   # block id names another K-block
    (None, True),                                                      # stored map is not the index's
])
def test_read_hypertensor_refuses_tampered_files(tmp_path, orc, tamper, fmt_tamper):
    p = str(tmp_path / "bad.safetensors")
    _write_packed_file(p, orc, tamper, fmt_tamper)
    with pytest.raises(ValueError):
        htnn.read_hypertensor(p)
