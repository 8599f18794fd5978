"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The GPU runs every row; the oracle checks a sample of outputs it can compute one by one (each
row's log-prob and entropy need only that row's logits; a grad_weight row needs every token's
log-sum-exp, i.e. one full oracle pass over the logits)."""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from oracle import fp64
from tests.gpu_util import (GRAD_REL_FRO, assert_entropy, assert_logprob, assert_softmax_rows, bits, dev,
                            label_rows, rel_fro)

pytestmark = pytest.mark.gpu


def _fwd_all(x):
    h, w, y = x.hidden.to(dev()), x.weight.to(dev()), x.labels.to(dev())
    lp, ent, lse = lmh.forward(h, w, y, entropy=True, want_lse=True)
    torch.cuda.synchronize()
    return h, w, y, lp, ent, lse


def test_T8192_H4096_V152064_peaked_sampled_rows():
    name = "fwd_T8192_H4096_V152064_peaked"
    print(f"[case] {name}", flush=True)
    x = synth.make_workload(name)
    _, _, _, lp, ent, _ = _fwd_all(x)
    ent_np = ent.cpu().double().numpy()
    T = x.hidden.shape[0]
    g = torch.Generator().manual_seed(1234)
    rand_rows = torch.randperm(T, generator=g)[:448].numpy()
    tiny_rows = np.argsort(ent_np)[:64]                 # the most peaked rows (smallest entropy)
    rows = np.unique(np.concatenate([rand_rows, tiny_rows]))
    ref = fp64.forward_rows(x.hidden, x.weight, x.labels, rows)
    print(f"rows {len(rows)}, min oracle entropy {ref['entropy'].min():.3e}", flush=True)
    assert_logprob(lp.cpu().double().numpy()[rows], ref["logprob"], name)
    assert_entropy(ent_np[rows], ref["entropy"], name)
    assert ref["entropy"].min() < 1e-3, "the peaked recipe should produce very small entropies"


@pytest.mark.parametrize("T", [16, 64, 256])
def test_small_T_H5120_V152064_all_rows(T):
    name = f"fwd_T{T}_H5120_V152064"
    print(f"[case] {name}", flush=True)
    x = synth.make_workload(name)
    _, _, _, lp, ent, lse = _fwd_all(x)
    ref = fp64.forward(x.hidden, x.weight, x.labels)
    assert_logprob(lp.cpu().double().numpy(), ref["logprob"], name)
    assert_entropy(ent.cpu().double().numpy(), ref["entropy"], name)


def test_small_T_rows_equal_large_T_rows():
    # the small-T tiles and the large-T tiles must give the same bits for the same row
    x = synth.make_workload("fwd_T256_H5120_V152064")
    h, w, y = x.hidden.to(dev()), x.weight.to(dev()), x.labels.to(dev())
    big = torch.cat([h, synth.hidden(1792, 5120, seed=7).to(dev())])
    bigy = torch.cat([y, synth.labels(1792, 152064, seed=7).to(dev())])
    a = lmh.forward(h[:16], w, y[:16], entropy=True, want_lse=True)
    b = lmh.forward(h, w, y, entropy=True, want_lse=True)
    c = lmh.forward(big, w, bigy, entropy=True, want_lse=True)
    torch.cuda.synchronize()
    for i in range(3):
        assert np.array_equal(bits(a[i]), bits(b[i][:16]))
        assert np.array_equal(bits(b[i]), bits(c[i][:256]))


def test_T4096_H5120_V152064_backward_sampled():
    name = "fwdbwd_T4096_H5120_V152064"
    print(f"[case] {name}", flush=True)
    x = synth.make_workload(name)
    h, w, y, lp, ent, lse = _fwd_all(x)
    g = x.grad.to(dev())
    gh, gw = lmh.backward(h, w, y, g, lse)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(99)
    trows = torch.randperm(x.hidden.shape[0], generator=gen)[:16].numpy()
    vrows = np.concatenate([torch.randperm(x.weight.shape[0], generator=gen)[:14].numpy(),
                            x.labels[:2].long().numpy()])       # include rows with label terms
    W64 = fp64.to_f64(x.weight)
    rgh = fp64.grad_hidden_rows(x.hidden, W64, x.labels, x.grad, trows)
    e1 = rel_fro(gh.cpu().double().numpy()[trows], rgh)
    print(f"grad_hidden rel fro on 16 rows {e1:.3e}", flush=True)
    rgw = fp64.grad_weight_rows(x.hidden, W64, x.labels, x.grad, vrows)
    e2 = rel_fro(gw.cpu().double().numpy()[vrows], rgw)
    print(f"grad_weight rel fro on 16 rows {e2:.3e}", flush=True)
    assert e1 <= GRAD_REL_FRO and e2 <= GRAD_REL_FRO
    # the sampled rows that hold no label carry only the softmax term: gated on their own
    is_label = label_rows(x.labels.numpy(), x.weight.shape[0])[vrows]
    assert_softmax_rows(gw.cpu().double().numpy()[vrows], rgw, is_label, name)

    # bitwise: grad_hidden rows do not depend on the batch split; grad_weight accumulated over a
    # split at a multiple of 64 tokens reproduces the single call
    half = x.hidden.shape[0] // 2
    gw2 = torch.empty_like(gw)
    parts = []
    for i, (s0, s1) in enumerate(((0, half), (half, x.hidden.shape[0]))):
        hs, ys, gs = h[s0:s1], y[s0:s1], g[s0:s1]
        _, _, lse_s = lmh.forward(hs, w, ys, want_lse=True)
        ghs = torch.empty((s1 - s0, h.shape[1]), dtype=torch.float32, device=dev())
        ws = torch.empty(lmh.lmhead_logprob_bwd_workspace_size(s1 - s0, h.shape[1], w.shape[0]), dtype=torch.uint8,
                         device=dev())
        lmh.lmhead_logprob_bwd(hs, w, ys, gs, lse_s, ghs, gw2, i > 0, ws)
        parts.append(ghs)
    torch.cuda.synchronize()
    assert np.array_equal(bits(torch.cat(parts)), bits(gh))
    assert np.array_equal(bits(gw2), bits(gw))

    # a 256 MB workspace (a 7936-row vocabulary step instead of 65536) gives the same bits
    T, H, V = x.hidden.shape[0], x.hidden.shape[1], x.weight.shape[0]
    assert lmh.lmhead_logprob_bwd_workspace_size(T, H, V) > 256 << 20
    ws = torch.empty(256 << 20, dtype=torch.uint8, device=dev())
    gh3 = torch.empty_like(gh)
    gw3 = torch.empty_like(gw)
    lmh.lmhead_logprob_bwd(h, w, y, g, lse, gh3, gw3, False, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(gh3), bits(gh)) and np.array_equal(bits(gw3), bits(gw))
