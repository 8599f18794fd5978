"""GPU parity of the extended entry points against the fp64 oracle: temperature, sum of squared
probabilities, the entropy gradient, and vocabulary shards folded after the fact.

Everything runs through the C ABI (the ``_ex`` entry points); the oracle is ``oracle.fp64`` with
the same fp32 temperature value."""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from oracle import fp64
from tests.gpu_util import GRAD_REL_FRO, assert_entropy, assert_logprob, bits, dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu

SUM_P2_RTOL = 1e-3   # sum_j p^2 lies in [1/V, 1]; fp32 records and fold give ~1e-6 relative error


def f32(x):
    return float(np.float32(x))


def _case(T, H, V, seed, wstd=0.05, peaked=0.0):
    x = synth.make_inputs(T, H, V, seed=seed, weight_std=wstd, peaked_frac=peaked, with_grad=True)
    return x.hidden, x.weight, x.labels, x.grad


def _fwd_ex(h, w, y, tau):
    """logprob, entropy, lse, sum_p2 through lmhead_logprob_fwd_ex (fp32 device tensors)."""
    out = lmh.forward(h, w, y, entropy=True, want_lse=True, temperature=tau, sum_p2=True)
    torch.cuda.synchronize()
    return out


def _np(t):
    return t.cpu().double().numpy()


@pytest.mark.parametrize("T,H,V,tau", [(37, 256, 4099, 0.7), (300, 520, 2053, 1.7), (17, 136, 1000, 0.25),
                                       (513, 128, 777, 3.0)])
def test_temperature_and_sum_p2_parity(T, H, V, tau):
    tau = f32(tau)
    print(f"[case] temperature {tau} T={T} H={H} V={V}", flush=True)
    h, w, y, _ = _case(T, H, V, seed=T, wstd=0.08)
    ref = fp64.forward(h, w, y, temperature=tau, sum_p2=True)
    lp, ent, lse, p2 = _fwd_ex(*to_dev(h, w, y), tau)
    assert_logprob(_np(lp), ref["logprob"], "temperature")
    assert_entropy(_np(ent), ref["entropy"], "temperature")
    np.testing.assert_allclose(_np(lse), ref["lse"], rtol=0, atol=2e-3 + 1e-6 * np.abs(ref["lse"]).max())
    np.testing.assert_allclose(_np(p2), ref["sum_p2"], rtol=SUM_P2_RTOL, atol=0)


def test_temperature_one_is_the_plain_path_bitwise():
    h, w, y, _ = to_dev(*_case(300, 256, 4099, seed=5))
    base = lmh.forward(h, w, y, entropy=True, want_lse=True)
    ex = lmh.forward(h, w, y, entropy=True, want_lse=True, temperature=1.0, sum_p2=True)
    torch.cuda.synchronize()
    for a, b in zip(base, ex[:3]):
        assert np.array_equal(bits(a), bits(b))


def test_fp32_temperature_is_not_rounded_to_bf16():
    # The pages' pitfall: a temperature cast to bf16 (0.7 -> 0.69921875) is a different input.
    h, w, y, _ = _case(256, 256, 4096, seed=8, wstd=0.3)
    tau, tau_bf16 = f32(0.7), 0.69921875
    lp, _, _, _ = _fwd_ex(*to_dev(h, w, y), tau)
    ref = fp64.forward(h, w, y, temperature=tau)["logprob"]
    ref_bf16 = fp64.forward(h, w, y, temperature=tau_bf16)["logprob"]
    assert_logprob(_np(lp), ref, "fp32 temperature")
    assert np.abs(_np(lp) - ref_bf16).max() > 2e-3


def test_peaked_rows_with_temperature_and_sum_p2():
    h, w, y, _ = _case(64, 256, 4096, seed=9, wstd=0.05, peaked=0.01)
    tau = f32(0.6)
    ref = fp64.forward(h, w, y, temperature=tau, sum_p2=True)
    lp, ent, _, p2 = _fwd_ex(*to_dev(h, w, y), tau)
    assert_logprob(_np(lp), ref["logprob"], "peaked")
    assert_entropy(_np(ent), ref["entropy"], "peaked")
    np.testing.assert_allclose(_np(p2), ref["sum_p2"], rtol=SUM_P2_RTOL, atol=0)


def test_temperature_rows_are_batch_invariant():
    h, w, y, _ = to_dev(*_case(300, 256, 4099, seed=10))
    tau = f32(0.8)
    full = _fwd_ex(h, w, y, tau)
    for c in (1, 7, 64):
        parts = [_fwd_ex(h[s:s + c], w, y[s:s + c], tau) for s in range(0, 300, c)]
        for k in range(4):
            assert np.array_equal(bits(torch.cat([p[k] for p in parts])), bits(full[k])), f"chunks of {c}, output {k}"


@pytest.mark.parametrize("order", ["ascending", "descending"])
@pytest.mark.parametrize("tau,T", [(1.0, 300), (0.9, 37)])
def test_vocabulary_shards_fold_to_the_single_call(order, tau, T):
    # Shards on 128-row chunks, run one after another into one workspace, then one fold: the same
    # bits as one call over the whole weight, in any shard order.
    tau = f32(tau)
    H, V = 256, 4099
    h, w, y, _ = to_dev(*_case(T, H, V, seed=11, wstd=0.08))
    y = y.clone()
    y[0] = -100
    ref = _fwd_ex(h, w, y, tau)
    bounds = [0, 1024, 1152, 3072, V]
    shards = list(zip(bounds[:-1], bounds[1:]))
    if order == "descending":
        shards = shards[::-1]
    ws = torch.empty(lmh.lmhead_logprob_fwd_workspace_size(T, H, V), dtype=torch.uint8, device=dev())
    for v0, v1 in shards:
        lmh.lmhead_logprob_fwd_partials_ex(h, w[v0:v1], y, tau, v0, V, True, ws)
    out = [torch.empty(T, dtype=torch.float32, device=dev()) for _ in range(4)]
    lmh.lmhead_logprob_fwd_finalize_ex(y, T, H, V, out[0], out[1], out[2], out[3], ws)
    torch.cuda.synchronize()
    for k in range(4):
        assert np.array_equal(bits(out[k]), bits(ref[k])), f"output {k}"


def test_shard_labels_outside_every_shard_give_zero():
    T, H, V = 70, 128, 1000
    h, w, y, _ = to_dev(*_case(T, H, V, seed=12))
    y = y.clone()
    y[0], y[1], y[2] = -1, V, 2**31 - 1
    ws = torch.empty(lmh.lmhead_logprob_fwd_workspace_size(T, H, V), dtype=torch.uint8, device=dev())
    for v0, v1 in ((0, 512), (512, V)):
        lmh.lmhead_logprob_fwd_partials_ex(h, w[v0:v1], y, 1.0, v0, V, False, ws)
    lp = torch.empty(T, dtype=torch.float32, device=dev())
    lmh.lmhead_logprob_fwd_finalize_ex(y, T, H, V, lp, None, None, None, ws)
    torch.cuda.synchronize()
    assert float(lp[0]) == 0.0 and float(lp[1]) == 0.0 and float(lp[2]) == 0.0
    ref = fp64.forward(h.cpu(), w.cpu(), y.cpu())
    assert_logprob(_np(lp), ref["logprob"], "shards")


@pytest.mark.parametrize("T,H,V,tau,egrad", [(64, 128, 1000, 0.7, False), (100, 192, 2053, 1.0, True),
                                             (257, 256, 4099, 1.3, True), (40, 64, 40000, 0.5, True)])
def test_backward_with_temperature_and_entropy_gradient(T, H, V, tau, egrad):
    tau = f32(tau)
    print(f"[case] bwd_ex T={T} H={H} V={V} tau={tau} entropy_grad={egrad}", flush=True)
    h, w, y, g = _case(T, H, V, seed=T + 1)
    y = y.clone()
    y[3] = -100
    ge = synth.upstream_grad(T, T + 2) if egrad else None
    hd, wd, yd, gd = to_dev(h, w, y, g)
    _, ent, lse = lmh.forward(hd, wd, yd, entropy=True, want_lse=True, temperature=tau)
    gh, gw = lmh.backward(hd, wd, yd, gd, lse, temperature=tau, grad_entropy=None if ge is None else ge.to(dev()),
                          entropy=ent)
    torch.cuda.synchronize()
    rgh, rgw = fp64.backward(h, w, y, g, temperature=tau, grad_entropy=ge)
    e1 = rel_fro(_np(gh), rgh)
    e2 = rel_fro(_np(gw), rgw)
    print(f"rel fro grad_hidden {e1:.3e} grad_weight {e2:.3e}", flush=True)
    assert e1 <= GRAD_REL_FRO and e2 <= GRAD_REL_FRO


@pytest.mark.parametrize("tau,egrad", [(1.0, False), (0.7, True)])
def test_backward_vocabulary_shards(tau, egrad):
    # Shards of the weight with the whole vocabulary's lse: each shard's grad_weight rows are the
    # bits of the whole call's rows, the grad_hidden shares add up to the whole call's, and every
    # share matches the oracle's share.  Shard starts need no alignment in the backward.
    tau = f32(tau)
    T, H, V = 100, 192, 3000
    print(f"[case] bwd_ex shards T={T} H={H} V={V} tau={tau} entropy_grad={egrad}", flush=True)
    h, w, y, g = _case(T, H, V, seed=31)
    y = y.clone()
    y[:3] = torch.tensor([5, 1500, 2999], dtype=y.dtype)
    y[3] = -100
    ge = synth.upstream_grad(T, 32) if egrad else None
    hd, wd, yd, gd = to_dev(h, w, y, g)
    ged = None if ge is None else ge.to(dev())
    _, ent, lse = lmh.forward(hd, wd, yd, entropy=True, want_lse=True, temperature=tau)
    gh, gw = lmh.backward(hd, wd, yd, gd, lse, temperature=tau, grad_entropy=ged, entropy=ent, vocab_start=0)
    bounds = [0, 1000, 1501, 2990, V]
    gh_sum = torch.zeros_like(gh)
    for v0, v1 in zip(bounds[:-1], bounds[1:]):
        ghs, gws = lmh.backward(hd, wd[v0:v1], yd, gd, lse, temperature=tau, grad_entropy=ged, entropy=ent,
                                vocab_start=v0)
        torch.cuda.synchronize()
        assert np.array_equal(bits(gws), bits(gw[v0:v1])), f"grad_weight rows of shard [{v0}, {v1})"
        rgh, rgw = fp64.backward_shard(h, w, y, g, v0, v1, temperature=tau, grad_entropy=ge)
        e1, e2 = rel_fro(_np(ghs), rgh), rel_fro(_np(gws), rgw)
        print(f"shard [{v0}, {v1}) rel fro grad_hidden {e1:.3e} grad_weight {e2:.3e}", flush=True)
        assert e1 <= GRAD_REL_FRO and e2 <= GRAD_REL_FRO
        gh_sum += ghs
    assert rel_fro(_np(gh_sum), _np(gh)) <= 1e-5


def test_entropy_only_gradient():
    # only the entropy carries a gradient: zero upstream gradient on the log-probs
    T, H, V = 64, 128, 2053
    h, w, y, _ = _case(T, H, V, seed=13)
    ge = synth.upstream_grad(T, 14)
    hd, wd, yd = to_dev(h, w, y)
    _, ent, lse = lmh.forward(hd, wd, yd, entropy=True, want_lse=True)
    gh, gw = lmh.backward(hd, wd, yd, torch.zeros(T, dtype=torch.float32, device=dev()), lse,
                          grad_entropy=ge.to(dev()), entropy=ent)
    torch.cuda.synchronize()
    rgh, rgw = fp64.backward(h, w, y, np.zeros(T), grad_entropy=ge)
    assert rel_fro(_np(gh), rgh) <= GRAD_REL_FRO and rel_fro(_np(gw), rgw) <= GRAD_REL_FRO


def test_autograd_through_logprob_and_entropy():
    T, H, V = 48, 128, 1000
    h, w, y, g = _case(T, H, V, seed=15)
    ge = synth.upstream_grad(T, 16)
    tau = f32(0.75)
    hd = h.to(dev()).float().requires_grad_(True)
    wd = w.to(dev()).requires_grad_(True)
    lp, ent = lmh.logprob(hd, wd, y.to(dev()), entropy=True, temperature=tau)
    loss = (lp * g.to(dev())).sum() + (ent * ge.to(dev())).sum()
    loss.backward()
    rgh, rgw = fp64.backward(h, w, y, g, temperature=tau, grad_entropy=ge)
    assert hd.grad.dtype == torch.float32 and wd.grad.dtype == torch.bfloat16
    assert rel_fro(_np(hd.grad), rgh) <= GRAD_REL_FRO
    assert rel_fro(_np(wd.grad), rgw) <= GRAD_REL_FRO   # returned in bf16, the weight's dtype


def test_full_size_temperature_sampled_rows():
    # T=2048 H=4096 V=152064 through the persistent large-T tile, temperature 0.7 and sum_p2
    name = "fwd_T2048_H4096_V152064"
    print(f"[case] {name} temperature 0.7", flush=True)
    x = synth.make_workload(name)
    tau = f32(0.7)
    lp, ent, _, p2 = _fwd_ex(*to_dev(x.hidden, x.weight, x.labels), tau)
    rows = torch.randperm(2048, generator=torch.Generator().manual_seed(5))[:96].numpy()
    ref = fp64.forward_rows(x.hidden, x.weight, x.labels, rows, temperature=tau, sum_p2=True)
    assert_logprob(_np(lp)[rows], ref["logprob"], name)
    assert_entropy(_np(ent)[rows], ref["entropy"], name)
    np.testing.assert_allclose(_np(p2)[rows], ref["sum_p2"], rtol=SUM_P2_RTOL, atol=0)


@pytest.mark.parametrize("T", [40, 300])
def test_sum_p2_without_recorded_squares_is_nan(T):
    # finalize asked for sum_p2 after a shard's partials ran without it: NaN in sum_p2 for every
    # row (the workspace's per-chunk flags), everything else as usual
    H, V = 64, 1000
    print(f"[case] sum_p2 guard T={T}", flush=True)
    h, w, y, _ = to_dev(*_case(T, H, V, seed=41))
    ws = torch.empty(lmh.lmhead_logprob_fwd_workspace_size(T, H, V), dtype=torch.uint8, device=dev())
    out = [torch.empty(T, dtype=torch.float32, device=dev()) for _ in range(4)]
    lmh.lmhead_logprob_fwd_partials_ex(h, w[:512], y, 1.0, 0, V, True, ws)
    lmh.lmhead_logprob_fwd_partials_ex(h, w[512:], y, 1.0, 512, V, False, ws)
    lmh.lmhead_logprob_fwd_finalize_ex(y, T, H, V, *out, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out[3]).all())
    ref = lmh.forward(h, w, y, entropy=True, want_lse=True)
    for i in range(3):
        assert np.array_equal(bits(out[i]), bits(ref[i]))
    # both shards with squared sums: finite and equal to the one-call value
    lmh.lmhead_logprob_fwd_partials_ex(h, w[512:], y, 1.0, 512, V, True, ws)
    lmh.lmhead_logprob_fwd_finalize_ex(y, T, H, V, *out, workspace=ws)
    one = lmh.forward(h, w, y, entropy=True, want_lse=True, sum_p2=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out[3]), bits(one[3]))


def test_autograd_wide_labels_take_the_out_of_range_rule():
    # int64 labels outside the int32 range must not wrap onto a vocabulary id (2^32 + 5 -> 5)
    T, H, V = 24, 128, 1000
    h, w, y, g = _case(T, H, V, seed=43)
    y64 = y.to(torch.int64)
    y64[:4] = torch.tensor([2**32 + 5, -(2**40), 2**31, V], dtype=torch.int64)
    y_ref = y.clone()
    y_ref[:4] = -1
    hd = h.to(dev()).float().requires_grad_(True)
    wd = w.to(dev()).requires_grad_(True)
    lp, _ = lmh.logprob(hd, wd, y64.to(dev()))
    (lp * g.to(dev())).sum().backward()
    assert bool((lp[:4] == 0).all())
    ref = fp64.forward(h, w, y_ref)
    assert_logprob(_np(lp.detach()), ref["logprob"], "wide labels")
    rgh, rgw = fp64.backward(h, w, y_ref, g)
    assert rel_fro(_np(hd.grad), rgh) <= GRAD_REL_FRO and rel_fro(_np(wd.grad), rgw) <= GRAD_REL_FRO
