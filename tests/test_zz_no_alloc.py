"""The allocation-free forward (lmhead_logprob_fwd_noalloc) against the workspace forward.

Both run the same kernels, so the outputs must be the same bits.  Two calls in a row, the second
with a smaller input (and a different tile family), check that the built-in scratch keeps no state
that matters between calls; an oversized call must be refused before anything is launched."""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from tests.gpu_util import bits, dev

pytestmark = pytest.mark.gpu


def _pair(T, H, V, seed):
    x = synth.make_inputs(T, H, V, seed=seed, weight_std=0.05)
    y = x.labels.clone()
    if T > 3:
        y[1] = -100
        y[2] = V
    h, w, yd = x.hidden.to(dev()), x.weight.to(dev()), y.to(dev())
    ref = lmh.forward(h, w, yd, entropy=True, want_lse=True)
    got = [torch.full((T,), float("nan"), dtype=torch.float32, device=dev()) for _ in range(3)]
    lmh.lmhead_logprob_fwd_noalloc(h, w, yd, got[0], got[1], got[2])
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("first,second", [((300, 256, 5000), (37, 136, 1000)),
                                          ((8192, 256, 4099), (5, 64, 300))])
def test_noalloc_matches_workspace_forward(first, second):
    for k, (T, H, V) in enumerate((first, second)):
        print(f"[case] noalloc call {k}: T={T} H={H} V={V}", flush=True)
        ref, got = _pair(T, H, V, seed=T + k)
        for i, name in enumerate(("logprob", "entropy", "lse")):
            assert np.array_equal(bits(got[i]), bits(ref[i])), f"call {k}: {name} differs from lmhead_logprob_fwd"


def test_noalloc_full_vocabulary_and_limit():
    # the largest T whose workspace fits the scratch at V = 152064, then one row more is refused
    H, V = 256, 152064
    fit = 1
    while lmh.lmhead_logprob_fwd_workspace_size_min(fit + 1, H, V) <= lmh.NOALLOC_SCRATCH_BYTES:
        fit += 1
    print(f"[case] noalloc at the limit: T={fit} H={H} V={V}", flush=True)
    ref, got = _pair(fit, H, V, seed=3)
    for i in range(3):
        assert np.array_equal(bits(got[i]), bits(ref[i]))
    T = fit + 1
    x = synth.make_inputs(T, H, V, seed=4)
    h, w, y = x.hidden.to(dev()), x.weight.to(dev()), x.labels.to(dev())
    lp = torch.full((T,), 7.0, dtype=torch.float32, device=dev())
    with pytest.raises(lmh.LmheadError) as e:
        lmh.lmhead_logprob_fwd_noalloc(h, w, y, lp)
    assert e.value.status == lmh.LMH_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((lp == 7.0).all()), "a refused call must launch nothing"
