"""The seeded input generator: determinism, shapes, ranges and the recipe's distributions."""
import math

import torch

import synth


def test_deterministic_and_streams_distinct():
    a = synth.make_inputs(32, 64, 300, seed=0, with_grad=True)
    b = synth.make_inputs(32, 64, 300, seed=0, with_grad=True)
    assert torch.equal(a.hidden.view(torch.int16), b.hidden.view(torch.int16))
    assert torch.equal(a.weight.view(torch.int16), b.weight.view(torch.int16))
    assert torch.equal(a.labels, b.labels) and torch.equal(a.grad, b.grad)
    c = synth.make_inputs(32, 64, 300, seed=1)
    assert not torch.equal(a.hidden.view(torch.int16), c.hidden.view(torch.int16))


def test_shapes_dtypes_ranges():
    x = synth.make_inputs(17, 40, 1000, seed=2, with_grad=True)
    assert x.hidden.shape == (17, 40) and x.hidden.dtype == torch.bfloat16
    assert x.weight.shape == (1000, 40) and x.weight.dtype == torch.bfloat16
    assert x.labels.dtype == torch.int32 and int(x.labels.min()) >= 0 and int(x.labels.max()) < 1000
    assert x.grad.dtype == torch.float32 and x.grad.shape == (17,)


def test_distribution_scales():
    h = synth.hidden(256, 512, 0).float()
    w = synth.weight(2048, 512, 0, 0.02).float()
    assert abs(h.std().item() - 1.0) < 0.02 and abs(h.mean().item()) < 0.02
    assert abs(w.std().item() - 0.02) < 0.0005


def test_peaked_rows():
    V, H = 5000, 64
    base = synth.weight(V, H, 4, 0.02).float()
    pk = synth.weight(V, H, 4, 0.02, peaked_frac=0.01).float()
    rows = synth.peaked_rows(V, 4, 0.01)
    assert rows.numel() == math.floor(0.01 * V)
    mask = torch.zeros(V, dtype=torch.bool)
    mask[rows] = True
    assert torch.equal(pk[~mask], base[~mask])
    ratio = pk[mask].norm() / base[mask].norm()
    assert abs(ratio.item() - 10.0) < 0.05


def test_workloads_named():
    w = synth.WORKLOADS["fwd_T8192_H4096_V152064_peaked"]
    assert (w.T, w.H, w.V, w.peaked_frac) == (8192, 4096, 152064, 0.01)
    assert synth.WORKLOADS["fwdbwd_T4096_H5120_V152064"].backward
