"""GPU backward parity against the fp64 oracle, plus determinism and split invariance."""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from oracle import fp64
from tests.gpu_util import GRAD_REL_FRO, assert_softmax_rows, bits, dev, label_rows, rel_fro, to_dev

pytestmark = pytest.mark.gpu


def _case(T, H, V, seed, wstd=0.05):
    x = synth.make_inputs(T, H, V, seed=seed, weight_std=wstd, with_grad=True)
    return x.hidden, x.weight, x.labels, x.grad


def _grads(h, w, y, g, acc_into=None):
    lp, _, lse = lmh.forward(h, w, y, want_lse=True)
    gh, gw = lmh.backward(h, w, y, g, lse)
    torch.cuda.synchronize()
    return gh, gw


# (40, 64, 140000) walks three 65536-row vocabulary steps, the last one ragged
@pytest.mark.parametrize("T,H,V", [(64, 128, 1000), (100, 192, 2053), (257, 256, 4099), (40, 64, 40000),
                                   (40, 64, 140000)])
def test_backward_parity(T, H, V):
    print(f"[case] bwd T={T} H={H} V={V}", flush=True)
    h, w, y, g = _case(T, H, V, seed=T)
    y = y.clone()
    y[3] = -100
    y[7] = V
    gh, gw = _grads(*to_dev(h, w, y, g))
    rgh, rgw = fp64.backward(h, w, y, g)
    e1 = rel_fro(gh.cpu().double().numpy(), rgh)
    e2 = rel_fro(gw.cpu().double().numpy(), rgw)
    print(f"rel fro grad_hidden {e1:.3e} grad_weight {e2:.3e}", flush=True)
    assert e1 <= GRAD_REL_FRO and e2 <= GRAD_REL_FRO
    assert_softmax_rows(gw.cpu().double().numpy(), rgw, label_rows(y.numpy(), V), f"{T}x{H}x{V}")


def test_zero_hidden_gives_zero_grad_weight():
    T, H, V = 50, 128, 777
    _, w, y, g = _case(T, H, V, seed=3)
    h = torch.zeros((T, H), dtype=torch.bfloat16)
    gh, gw = _grads(*to_dev(h, w, y, g))
    assert torch.count_nonzero(gw).item() == 0
    rgh, _ = fp64.backward(h, w, y, g)
    assert rel_fro(gh.cpu().double().numpy(), rgh) <= GRAD_REL_FRO


def test_grad_hidden_split_invariance_and_repeat():
    T, H, V = 300, 256, 20000
    h, w, y, g = to_dev(*_case(T, H, V, seed=11))
    gh, gw = _grads(h, w, y, g)
    gh2, gw2 = _grads(h, w, y, g)
    assert np.array_equal(bits(gh), bits(gh2)) and np.array_equal(bits(gw), bits(gw2))
    parts = []
    for s in range(0, T, 37):
        p, _ = _grads(h[s:s + 37], w, y[s:s + 37], g[s:s + 37])
        parts.append(bits(p))
    assert np.array_equal(np.concatenate(parts), bits(gh))


def test_grad_weight_split_accumulate_is_bitwise():
    T, H, V = 320, 128, 3000
    h, w, y, g = to_dev(*_case(T, H, V, seed=12))
    _, gw = _grads(h, w, y, g)
    acc = torch.empty_like(gw)
    for i, s in enumerate(range(0, T, 128)):
        hs, ys, gs = h[s:s + 128], y[s:s + 128], g[s:s + 128]
        _, _, lse = lmh.forward(hs, w, ys, want_lse=True)
        ws = torch.empty(lmh.lmhead_logprob_bwd_workspace_size(hs.shape[0], H, V), dtype=torch.uint8, device=dev())
        lmh.lmhead_logprob_bwd(hs, w, ys, gs, lse, None, acc, i > 0, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(acc), bits(gw))


def _bwd_with_workspace(h, w, y, g, lse, nbytes):
    T, H = h.shape
    V = w.shape[0]
    gh = torch.empty((T, H), dtype=torch.float32, device=dev())
    gw = torch.empty((V, H), dtype=torch.float32, device=dev())
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev())
    lmh.lmhead_logprob_bwd(h, w, y, g, lse, gh, gw, False, ws)
    torch.cuda.synchronize()
    return bits(gh), bits(gw)


@pytest.mark.parametrize("T,H,V", [(300, 256, 5000), (40, 64, 140000)])
def test_step_width_does_not_change_bits(T, H, V):
    # the workspace decides the vocabulary step (the widest multiple of 256 that fits); every step
    # width must give the bits of the widest
    print(f"[case] bwd step widths T={T} H={H} V={V}", flush=True)
    h, w, y, g = to_dev(*_case(T, H, V, seed=T + 5))
    _, _, lse = lmh.forward(h, w, y, want_lse=True)
    ref = _bwd_with_workspace(h, w, y, g, lse, lmh.lmhead_logprob_bwd_workspace_size(T, H, V))
    for step in (256, 768, 4096, 33024):
        got = _bwd_with_workspace(h, w, y, g, lse, lmh.lmhead_logprob_bwd_workspace_size_step(T, H, V, step))
        assert np.array_equal(got[0], ref[0]), f"grad_hidden differs at step {step}"
        assert np.array_equal(got[1], ref[1]), f"grad_weight differs at step {step}"
