"""Bitwise batch invariance of the forward on the GPU (no oracle needed): the same rows give the
same fp32 bits for logprob, entropy and lse whatever the batch size, their position in the batch,
or how the rows are split across calls.  The probe rows also go through the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import fp64
from tests.gpu_util import assert_entropy, assert_logprob, bits, dev, fwd_raw

pytestmark = pytest.mark.gpu

H, V = 4096, 152064
N_PROBE = 256


@pytest.fixture(scope="module")
def data():
    print("[setup] generating weight 152064 x 4096", flush=True)
    w = synth.weight(V, H, seed=0)
    probes = synth.hidden(N_PROBE, H, seed=20)
    py = synth.labels(N_PROBE, V, seed=20)
    filler = synth.hidden(2048, H, seed=21)
    fy = synth.labels(2048, V, seed=21)
    return dict(w_cpu=w, w=w.to(dev()), probes=probes.to(dev()), py=py.to(dev()), filler=filler.to(dev()),
                fy=fy.to(dev()), probes_cpu=probes, py_cpu=py)


def _outs(lp, ent, lse):
    return np.stack([bits(lp), bits(ent), bits(lse)], 1)


@pytest.fixture(scope="module")
def reference(data):
    """All probes in one call of T = 256 (in order)."""
    lp, ent, lse = fwd_raw(data["probes"], data["w"], data["py"])
    return _outs(lp, ent, lse), (lp, ent, lse)


def test_probe_parity_against_oracle(data, reference):
    idx = np.arange(N_PROBE)  # every probe row (about 0.3 TFLOP of fp64 work for the oracle)
    ref = fp64.forward_rows(data["probes_cpu"], data["w_cpu"], data["py_cpu"], idx)
    lp, ent, lse = [t.cpu().double().numpy()[idx] for t in reference[1]]
    assert_logprob(lp, ref["logprob"], "probes")
    assert_entropy(ent, ref["entropy"], "probes")


def test_single_row_batches(data, reference):
    got = []
    for i in range(N_PROBE):
        lp, ent, lse = fwd_raw(data["probes"][i:i + 1], data["w"], data["py"][i:i + 1])
        got.append(_outs(lp, ent, lse))
    got = np.concatenate(got)
    mism = int((got != reference[0]).any(1).sum())
    assert mism == 0, f"{mism} of {N_PROBE} rows differ bitwise at T=1"


def test_batches_of_seven(data, reference):
    g = synth.placement(N_PROBE, 7 * N_PROBE, seed=3)
    rows = []
    for i in range(N_PROBE):
        pos = int(g[i]) % 7
        h = data["filler"][7 * i % 2000: 7 * i % 2000 + 7].clone()
        y = data["fy"][7 * i % 2000: 7 * i % 2000 + 7].clone()
        h[pos] = data["probes"][i]
        y[pos] = data["py"][i]
        lp, ent, lse = fwd_raw(h, data["w"], y)
        rows.append(_outs(lp, ent, lse)[pos:pos + 1])
    got = np.concatenate(rows)
    mism = int((got != reference[0]).any(1).sum())
    assert mism == 0, f"{mism} of {N_PROBE} rows differ bitwise at T=7"


def test_permuted_batch(data, reference):
    perm = synth.placement(N_PROBE, N_PROBE, seed=4)
    lp, ent, lse = fwd_raw(data["probes"][perm.to(dev())].contiguous(), data["w"], data["py"][perm.to(dev())].contiguous())
    got = _outs(lp, ent, lse)
    inv = np.empty(N_PROBE, dtype=np.int64)
    inv[perm.numpy()] = np.arange(N_PROBE)
    mism = int((got[inv] != reference[0]).any(1).sum())
    assert mism == 0, f"{mism} rows differ bitwise after a permutation"


def test_embedded_in_2048(data, reference):
    pos = synth.placement(N_PROBE, 2048, seed=5).to(dev())
    h = data["filler"].clone()
    y = data["fy"].clone()
    h[pos] = data["probes"]
    y[pos] = data["py"]
    lp, ent, lse = fwd_raw(h, data["w"], y)
    got = _outs(lp, ent, lse)[pos.cpu().numpy()]
    mism = int((got != reference[0]).any(1).sum())
    assert mism == 0, f"{mism} rows differ bitwise inside a batch of 2048"


@pytest.mark.parametrize("c", [1, 3, 7, 16, 32, 64, 96, 128])
def test_row_chunk_sweep(data, reference, c):
    parts = []
    for s in range(0, N_PROBE, c):
        lp, ent, lse = fwd_raw(data["probes"][s:s + c], data["w"], data["py"][s:s + c])
        parts.append(_outs(lp, ent, lse))
    got = np.concatenate(parts)
    mism = int((got != reference[0]).any(1).sum())
    assert mism == 0, f"{mism} rows differ bitwise with row chunks of {c}"


def test_prime_length_chunks(data, reference):
    parts = []
    for s in range(0, 17, 5):
        e = min(17, s + 5)
        lp, ent, lse = fwd_raw(data["probes"][s:e], data["w"], data["py"][s:e])
        parts.append(_outs(lp, ent, lse))
    got = np.concatenate(parts)
    assert got.shape[0] == 17
    assert np.array_equal(got, reference[0][:17])


def test_repeat_run_identity(data, reference):
    for _ in range(3):
        lp, ent, lse = fwd_raw(data["probes"], data["w"], data["py"])
        assert np.array_equal(_outs(lp, ent, lse), reference[0])


@pytest.mark.parametrize("tau,p2", [(1.0, False), (0.7, True)])
def test_wave_fold_equals_block_fold(tau, p2):
    # T <= 512 folds one wavefront per row, larger T folds in row blocks: the same rows, alone and
    # inside a batch of 700, give the same bits (with a temperature and sum_p2 too)
    import lm_head_log_lmhead_amd as lmh
    H, V = 264, 20000
    x = synth.make_inputs(700, H, V, seed=31, weight_std=0.05)
    h, w, y = x.hidden.to(dev()), x.weight.to(dev()), x.labels.to(dev())
    big = lmh.forward(h, w, y, entropy=True, want_lse=True, temperature=tau, sum_p2=p2)
    for s0, s1 in ((0, 1), (5, 21), (100, 356), (400, 600)):
        part = lmh.forward(h[s0:s1], w, y[s0:s1], entropy=True, want_lse=True, temperature=tau, sum_p2=p2)
        torch.cuda.synchronize()
        for k in range(len(part)):
            assert np.array_equal(bits(part[k]), bits(big[k][s0:s1])), f"rows [{s0}, {s1}) output {k}"
