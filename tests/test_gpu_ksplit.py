"""The K-split schedule of the large-T forward tile (few tiles per compute unit: the K steps of
all tiles cut into equal ranges, accumulators handed between workgroups) against the dynamic
schedule of whole tiles: bit for bit, since every output's MFMA chain is the same.  The smallest
accepted workspace (lmhead_logprob_fwd_workspace_size_min) has no room for the split and runs the
dynamic schedule; the default size runs the split where it applies.  A sample of rows also goes
through the oracle."""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from oracle import fp64
from tests.gpu_util import assert_entropy, assert_logprob, bits, dev

pytestmark = pytest.mark.gpu


def _run(h, w, y, T, H, V, tau, p2, ws_bytes):
    lp, ent, lse = (torch.empty(T, dtype=torch.float32, device=dev()) for _ in range(3))
    sp = torch.empty(T, dtype=torch.float32, device=dev()) if p2 else None
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev())
    lmh.lmhead_logprob_fwd_ex(h, w, y, tau, lp, ent, lse, sp, ws)
    torch.cuda.synchronize()
    outs = [lp, ent, lse] + ([sp] if p2 else [])
    return np.stack([bits(t) for t in outs], 1), lp, ent


# (T, H, V, temperature, sum_p2), one token tile each:
#   274 vocabulary tiles of 5 steps on 256 workgroups: ranges of 5.35 steps, a split in almost every one;
#   274 tiles of 3 steps, the last one partial (H = 136), with a temperature and sum_p2 (T = 193);
#   274 tiles of 1 step (H = 64): ranges of whole tiles, no split;
#   the T = 256, H = 5120, V = 152064 workload: 594 tiles of 80 steps.
CASES = [(200, 264, 70000, 1.0, False), (193, 136, 70000, 0.7, True), (256, 64, 70000, 1.0, False),
         (256, 5120, 152064, 1.0, False)]


@pytest.mark.parametrize("T,H,V,tau,p2", CASES)
def test_ksplit_equals_whole_tiles(T, H, V, tau, p2):
    fast, least = lmh.lmhead_logprob_fwd_workspace_size(T, H, V), lmh.lmhead_logprob_fwd_workspace_size_min(T, H, V)
    assert fast > least, "the split applies to this shape"
    print(f"[case] ksplit T={T} H={H} V={V} tau={tau} p2={p2}", flush=True)
    x = synth.make_inputs(T, H, V, seed=T + H, weight_std=0.05)
    h, w, y = x.hidden.to(dev()), x.weight.to(dev()), x.labels.to(dev())
    split, lp, ent = _run(h, w, y, T, H, V, tau, p2, fast)
    again, _, _ = _run(h, w, y, T, H, V, tau, p2, fast)
    whole, _, _ = _run(h, w, y, T, H, V, tau, p2, least)
    assert np.array_equal(split, again), "repeat run"
    bad = np.nonzero((split != whole).any(1))[0]
    assert bad.size == 0, f"{bad.size} rows differ from the whole-tile schedule, first {bad[:8]}"
    rows = np.unique(np.linspace(0, T - 1, 12).astype(int))
    ref = fp64.forward_rows(x.hidden, x.weight, x.labels, rows=rows, temperature=tau)
    assert_logprob(lp.cpu().double().numpy()[rows], ref["logprob"], f"ksplit {T}x{H}x{V}")
    assert_entropy(ent.cpu().double().numpy()[rows], ref["entropy"], f"ksplit {T}x{H}x{V}")


def test_ksplit_shard():
    # a vocabulary shard with the split (its own tile count decides) folds with another shard run
    # without it into the bits of one whole call
    T, H, V = 200, 136, 140000
    x = synth.make_inputs(T, H, V, seed=9, weight_std=0.05)
    h, w, y = x.hidden.to(dev()), x.weight.to(dev()), x.labels.to(dev())
    print(f"[case] ksplit shards T={T} H={H} V={V}", flush=True)
    one = lmh.forward(h, w, y, entropy=True, want_lse=True)
    ws = torch.empty(lmh.lmhead_logprob_fwd_workspace_size(T, H, V), dtype=torch.uint8, device=dev())
    least = lmh.lmhead_logprob_fwd_workspace_size_min(T, H, V)
    assert ws.numel() > least
    cut = 70016  # a multiple of 128: 274 and 274 vocabulary tiles
    for v0, v1, nbytes in ((0, cut, ws.numel()), (cut, V, least)):
        lmh.lmhead_logprob_fwd_partials_ex(h, w[v0:v1].contiguous(), y, 1.0, v0, V, False, ws[:nbytes])
    lp, ent, lse = (torch.empty(T, dtype=torch.float32, device=dev()) for _ in range(3))
    lmh.lmhead_logprob_fwd_finalize_ex(y, T, H, V, lp, ent, lse, None, ws)
    torch.cuda.synchronize()
    for k, t in enumerate((lp, ent, lse)):
        assert np.array_equal(bits(t), bits(one[k])), f"output {k}"


def test_ksplit_wait_timeout_gives_nan(monkeypatch):
    # A tail whose wait for the previous workgroup's accumulators runs out continues NaN
    # accumulators instead of stale ones.  LMH_SK_SPIN_LIMIT=0 makes every tail give up at once:
    # every row then folds a NaN record and all outputs are NaN (the log-prob of a label outside
    # the vocabulary stays 0); without it the call is back to its bits.
    T, H, V = 200, 264, 70000
    fast = lmh.lmhead_logprob_fwd_workspace_size(T, H, V)
    assert fast > lmh.lmhead_logprob_fwd_workspace_size_min(T, H, V), "the split applies to this shape"
    print(f"[case] ksplit timeout T={T} H={H} V={V}", flush=True)
    x = synth.make_inputs(T, H, V, seed=5, weight_std=0.05)
    h, w, y = x.hidden.to(dev()), x.weight.to(dev()), x.labels.to(dev())
    normal, _, _ = _run(h, w, y, T, H, V, 1.0, False, fast)
    monkeypatch.setenv("LMH_SK_SPIN_LIMIT", "0")
    _, lp, ent = _run(h, w, y, T, H, V, 1.0, False, fast)
    monkeypatch.delenv("LMH_SK_SPIN_LIMIT")
    lab = x.labels.numpy()
    inv = (lab >= 0) & (lab < V)
    lp, ent = lp.cpu().numpy(), ent.cpu().numpy()
    assert np.isnan(ent).all(), "entropy"
    assert np.isnan(lp[inv]).all() and (lp[~inv] == 0).all(), "logprob"
    again, _, _ = _run(h, w, y, T, H, V, 1.0, False, fast)
    assert np.array_equal(again, normal)
    # a value that is not a number keeps the default bound
    monkeypatch.setenv("LMH_SK_SPIN_LIMIT", "none")
    other, _, _ = _run(h, w, y, T, H, V, 1.0, False, fast)
    monkeypatch.delenv("LMH_SK_SPIN_LIMIT")
    assert np.array_equal(other, normal)
