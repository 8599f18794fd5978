"""GPU parity at the edges of the supported range: the largest hidden size (H = 2^20, a K loop of
16384 steps), the largest token count of the backward (T = 2^22 - 1), a vocabulary of 2^24 + 77
and temperatures far from 1, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from oracle import fp64
from tests.gpu_util import GRAD_REL_FRO, assert_entropy, assert_logprob, dev, rel_fro, to_dev

pytestmark = pytest.mark.gpu

SUM_P2_RTOL = 1e-3


def _np(t):
    return t.cpu().double().numpy()


def test_maximum_hidden_size():
    # weight std 0.002 keeps |z| ~ 2, so the fp32 chain over 2^20 products stays well inside the
    # 2e-3 log-prob gate; V = 200 leaves a ragged second vocabulary tile
    T, H, V = 3, 1 << 20, 200
    print(f"[case] T={T} H={H} V={V}", flush=True)
    x = synth.make_inputs(T, H, V, seed=51, weight_std=0.002, with_grad=True)
    h, w, y, g = to_dev(x.hidden, x.weight, x.labels, x.grad)
    lp, ent, lse = lmh.forward(h, w, y, entropy=True, want_lse=True)
    gh, gw = lmh.backward(h, w, y, g, lse)
    torch.cuda.synchronize()
    ref = fp64.forward(x.hidden, x.weight, x.labels)
    assert_logprob(_np(lp), ref["logprob"], "H = 2^20")
    assert_entropy(_np(ent), ref["entropy"], "H = 2^20")
    rgh, rgw = fp64.backward(x.hidden, x.weight, x.labels, x.grad)
    e1, e2 = rel_fro(_np(gh), rgh), rel_fro(_np(gw), rgw)
    print(f"rel fro grad_hidden {e1:.3e} grad_weight {e2:.3e}", flush=True)
    assert e1 <= GRAD_REL_FRO and e2 <= GRAD_REL_FRO


@pytest.mark.parametrize("tau", [0.01, 100.0])
def test_temperatures_far_from_one(tau):
    # 0.01 makes nearly one-hot rows (log-probs in the hundreds), 100 nearly uniform ones
    T, H, V = 37, 256, 4099
    tau = float(np.float32(tau))
    print(f"[case] temperature {tau} T={T} H={H} V={V}", flush=True)
    x = synth.make_inputs(T, H, V, seed=52, weight_std=0.05, with_grad=True)
    ge = synth.upstream_grad(T, 53)
    h, w, y, g = to_dev(x.hidden, x.weight, x.labels, x.grad)
    lp, ent, lse, p2 = lmh.forward(h, w, y, entropy=True, want_lse=True, temperature=tau, sum_p2=True)
    gh, gw = lmh.backward(h, w, y, g, lse, temperature=tau, grad_entropy=ge.to(dev()), entropy=ent)
    torch.cuda.synchronize()
    ref = fp64.forward(x.hidden, x.weight, x.labels, temperature=tau, sum_p2=True)
    assert_logprob(_np(lp), ref["logprob"], f"temperature {tau}")
    assert_entropy(_np(ent), ref["entropy"], f"temperature {tau}")
    np.testing.assert_allclose(_np(p2), ref["sum_p2"], rtol=SUM_P2_RTOL, atol=0)
    rgh, rgw = fp64.backward(x.hidden, x.weight, x.labels, x.grad, temperature=tau, grad_entropy=ge)
    e1, e2 = rel_fro(_np(gh), rgh), rel_fro(_np(gw), rgw)
    print(f"rel fro grad_hidden {e1:.3e} grad_weight {e2:.3e}", flush=True)
    assert e1 <= GRAD_REL_FRO and e2 <= GRAD_REL_FRO


def test_maximum_token_count():
    # T = 2^22 - 1, the largest the backward accepts: 16384 persistent forward tiles, a fold grid of
    # 131072 workgroups, dz^T rows of 2^22 tokens (a 256-row tile spans exactly 2^31 bytes) and a
    # grad_weight chain of 65536 K steps.  Forward and grad_hidden on sampled rows, grad_weight in
    # full, and a row split that must give the same bits.
    T, H, V = (1 << 22) - 1, 8, 130
    print(f"[case] T={T} H={H} V={V}", flush=True)
    x = synth.make_inputs(T, H, V, seed=54, weight_std=0.5, with_grad=True)
    h, w, y, g = to_dev(x.hidden, x.weight, x.labels, x.grad)
    lp, ent, lse = lmh.forward(h, w, y, entropy=True, want_lse=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(54).integers(0, T, 4000), [0, T - 1]]))
    ref = fp64.forward_rows(x.hidden, x.weight, x.labels, rows)
    assert_logprob(_np(lp)[rows], ref["logprob"], "T = 2^22 - 1")
    assert_entropy(_np(ent)[rows], ref["entropy"], "T = 2^22 - 1")
    s = 3 * T // 7
    parts = [lmh.forward(h[a:b], w, y[a:b], entropy=True, want_lse=True) for a, b in ((0, s), (s, T))]
    torch.cuda.synchronize()
    for k, full in enumerate((lp, ent, lse)):
        joined = torch.cat([p[k] for p in parts])
        assert torch.equal(joined.view(torch.int32), full.view(torch.int32)), f"output {k} changes with the split"
    del parts
    gh, gw = lmh.backward(h, w, y, g, lse)
    torch.cuda.synchronize()
    rgh = fp64.grad_hidden_rows(x.hidden, x.weight, x.labels, x.grad, rows)
    rgw = fp64.grad_weight_rows(x.hidden, x.weight, x.labels, x.grad, np.arange(V), row_block=1 << 16)
    e1, e2 = rel_fro(_np(gh)[rows], rgh), rel_fro(_np(gw), rgw)
    print(f"rel fro grad_hidden {e1:.3e} grad_weight {e2:.3e}", flush=True)
    assert e1 <= GRAD_REL_FRO and e2 <= GRAD_REL_FRO


def test_large_vocabulary():
    # V = 2^24 + 77: 131073 record chunks per row (fold segments of ~2048 chunks), 131074 large-T
    # tiles at T = 300, and 257 vocabulary steps in the backward.  The oracle sees sampled rows in
    # small blocks (a row of fp64 logits is 134 MB).
    H, V = 8, (1 << 24) + 77
    T = 300
    print(f"[case] T={T} H={H} V={V}", flush=True)
    x = synth.make_inputs(T, H, V, seed=55, weight_std=0.5, with_grad=True)
    h, w, y, g = to_dev(x.hidden, x.weight, x.labels, x.grad)
    lp, ent, lse = lmh.forward(h, w, y, entropy=True, want_lse=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(55).integers(0, T, 24), [0, T - 1]]))
    ref = fp64.forward_rows(x.hidden, x.weight, x.labels, rows, row_block=4)
    assert_logprob(_np(lp)[rows], ref["logprob"], "V = 2^24 + 77")
    assert_entropy(_np(ent)[rows], ref["entropy"], "V = 2^24 + 77")
    np.testing.assert_allclose(_np(lse)[rows], ref["lse"], rtol=0, atol=2e-3 + 1e-6 * np.abs(ref["lse"]).max())
    # backward on three rows: all of grad_hidden, sampled grad_weight rows (including the labels')
    t3 = slice(0, 3)
    gh, gw = lmh.backward(h[t3], w, y[t3], g[t3], lse[t3])
    torch.cuda.synchronize()
    vr = np.unique(np.concatenate([np.random.default_rng(56).integers(0, V, 2000), x.labels[:3].numpy(), [V - 1]]))
    rgh = fp64.grad_hidden_rows(x.hidden[t3], x.weight, x.labels[t3], x.grad[t3], np.arange(3), row_block=1)
    rgw = fp64.grad_weight_rows(x.hidden[t3], x.weight, x.labels[t3], x.grad[t3], vr, row_block=1)
    e1, e2 = rel_fro(_np(gh), rgh), rel_fro(_np(gw)[vr], rgw)
    print(f"rel fro grad_hidden {e1:.3e} grad_weight (sampled rows) {e2:.3e}", flush=True)
    assert e1 <= GRAD_REL_FRO and e2 <= GRAD_REL_FRO


def test_empty_batch_through_autograd():
    # T = 0: empty outputs, an empty grad_hidden and a zero grad_weight (the library launches
    # nothing and leaves gradient buffers untouched, so the binding hands out zeros)
    H, V = 64, 300
    print(f"[case] T=0 H={H} V={V}", flush=True)
    x = synth.make_inputs(1, H, V, seed=57, weight_std=0.05)
    h = x.hidden.to(dev())[:0].float().requires_grad_(True)
    w = x.weight.to(dev()).requires_grad_(True)
    y = x.labels.to(dev())[:0]
    lp, ent = lmh.logprob(h, w, y, entropy=True)
    assert lp.shape == (0,) and ent.shape == (0,)
    (lp.sum() + ent.sum()).backward()
    torch.cuda.synchronize()
    assert h.grad.shape == (0, H)
    assert torch.count_nonzero(w.grad).item() == 0


# one token count per forward tile: 32-token, 64-token and 128-token tiles, the K-split schedule
# (T = 200: 274 vocabulary tiles on at most 256 workgroups) and the dynamic 256 x 256 schedule
@pytest.mark.parametrize("T", [7, 50, 100, 200, 300])
def test_nan_inputs_reach_the_outputs(T):
    # A NaN logit makes its row's softmax NaN (the definition's max and sum are NaN), also when a
    # whole 128-row vocabulary chunk is NaN (no entry then equals the chunk's max); the other rows
    # of the batch are untouched.
    H, V = 136, 70000
    print(f"[case] nan T={T} H={H} V={V}", flush=True)
    x = synth.make_inputs(T, H, V, seed=T + 7)
    wn = x.weight.clone()
    wn[256:384] = float("nan")                       # vocabulary chunk 2, for every token
    hn = x.hidden.clone()
    bad_row = T // 2
    hn[bad_row] = float("nan")                       # one token's logits, every chunk
    for what, h_in, w_in in (("weight chunk", x.hidden, wn), ("hidden row", hn, x.weight)):
        h, w, y = to_dev(h_in, w_in, x.labels)
        lp, ent, lse = lmh.forward(h, w, y, entropy=True, want_lse=True)
        torch.cuda.synchronize()
        ref = fp64.forward(h_in, w_in, x.labels)
        for name, got, want in (("logprob", _np(lp), ref["logprob"]), ("entropy", _np(ent), ref["entropy"]),
                                ("lse", _np(lse), ref["lse"])):
            assert np.array_equal(np.isnan(got), np.isnan(want)), f"{what}: NaN pattern of {name}"
        ok = ~np.isnan(ref["lse"])
        assert ok.sum() == (0 if what == "weight chunk" else T - 1), what
        assert_logprob(_np(lp)[ok], ref["logprob"][ok], what)
        assert_entropy(_np(ent)[ok], ref["entropy"][ok], what)
    # the rows next to the NaN row have the clean batch's bits
    h, w, y = to_dev(x.hidden, x.weight, x.labels)
    clean = lmh.forward(h, w, y, entropy=True, want_lse=True)
    h, w, y = to_dev(hn, x.weight, x.labels)
    dirty = lmh.forward(h, w, y, entropy=True, want_lse=True)
    torch.cuda.synchronize()
    keep = np.arange(T) != bad_row
    for c, d in zip(clean, dirty):
        assert np.array_equal(c.cpu().view(torch.int32).numpy()[keep], d.cpu().view(torch.int32).numpy()[keep])
