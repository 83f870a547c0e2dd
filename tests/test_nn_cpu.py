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
