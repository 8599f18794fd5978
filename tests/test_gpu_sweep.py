"""GPU parity over a seeded random sweep of shapes and options, drawn rather than hand-picked.

Each case draws T (in the small-, mid- and large-tile ranges), H (any multiple of 8 from 8 to
640, so K can be shorter than one 64-wide step), V (1 to 4999, ragged against every tile) and
whether a temperature and sum_p2 are asked for, plants two out-of-range labels, and checks
through the C ABI, element by element against the fp64 oracle: log-prob, entropy, lse, sum_p2,
and both gradients (grad_weight rows that hold no label also on their own).  It also checks that
splitting the rows at a drawn point into two calls gives the same bits as one call.  Sizes keep the oracle to a fraction of a second per case."""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from oracle import fp64
from tests.gpu_util import (GRAD_REL_FRO, assert_entropy, assert_logprob, assert_softmax_rows, bits, label_rows,
                            rel_fro, to_dev)

pytestmark = pytest.mark.gpu

SUM_P2_RTOL = 1e-3


def _cases(n=16, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        lo, hi = [(1, 65), (65, 129), (129, 700)][i % 3]
        T = int(rng.integers(lo, hi))
        H = 8 * int(rng.integers(1, 4 if i % 5 == 0 else 81))   # every fifth case: H of 8 to 24
        V = int(rng.integers(1, 5000))
        tau = 1.0 if rng.random() < 0.5 else float(np.float32(rng.uniform(0.3, 3.0)))
        p2 = bool(rng.random() < 0.5)
        split = int(rng.integers(1, T)) if T > 1 else 0
        out.append((i, T, H, V, tau, p2, split))
    return out


CASES = _cases()


def _fwd(h, w, y, tau, p2):
    out = lmh.forward(h, w, y, entropy=True, want_lse=True, temperature=tau, sum_p2=p2)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("i,T,H,V,tau,p2,split", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_case(i, T, H, V, tau, p2, split):
    print(f"[case] sweep {i}: T={T} H={H} V={V} tau={tau} sum_p2={p2} split={split}", flush=True)
    x = synth.make_inputs(T, H, V, seed=100 + i, weight_std=0.05, with_grad=True)
    y = x.labels.clone()
    if T > 3:
        y[1] = -100
        y[T // 2] = V
    ref = fp64.forward(x.hidden, x.weight, y, temperature=tau, sum_p2=p2)
    h, w, yd, g = to_dev(x.hidden, x.weight, y, x.grad)
    out = _fwd(h, w, yd, tau, p2)
    lp, ent, lse = out[:3]
    assert_logprob(lp.cpu().double().numpy(), ref["logprob"], f"sweep {i}")
    assert_entropy(ent.cpu().double().numpy(), ref["entropy"], f"sweep {i}")
    np.testing.assert_allclose(lse.cpu().double().numpy(), ref["lse"], rtol=0,
                               atol=2e-3 + 1e-6 * np.abs(ref["lse"]).max())
    if p2:
        np.testing.assert_allclose(out[3].cpu().double().numpy(), ref["sum_p2"], rtol=SUM_P2_RTOL, atol=1e-7)

    if split:
        parts = [_fwd(h[a:b], w, yd[a:b], tau, p2) for a, b in ((0, split), (split, T))]
        for k in range(len(out)):
            joined = torch.cat([p[k] for p in parts])
            assert np.array_equal(bits(joined), bits(out[k])), f"sweep {i}: output {k} changes with the row split"

    gh, gw = lmh.backward(h, w, yd, g, lse, temperature=tau)
    torch.cuda.synchronize()
    rgh, rgw = fp64.backward(x.hidden, x.weight, y, x.grad, temperature=tau)
    assert rel_fro(gh.cpu().double().numpy(), rgh) <= GRAD_REL_FRO, f"sweep {i} grad_hidden"
    assert rel_fro(gw.cpu().double().numpy(), rgw) <= GRAD_REL_FRO, f"sweep {i} grad_weight"
    is_label = label_rows(y.numpy(), V)
    if not is_label.all():
        assert_softmax_rows(gw.cpu().double().numpy(), rgw, is_label, f"sweep {i}")
