"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

The pages print no log-prob or entropy values for any input, so the oracle is pinned by
mathematics: an independent scalar implementation with correctly rounded sums, closed forms,
invariants, special cases and finite differences.  Each pin is chosen so that a plausible slip
(a dropped term, a sign, an index, a transposed operand) breaks at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import brute, fp64


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _rand_case(T, H, V, seed, hstd=1.0, wstd=0.3):
    h = synth.hidden(T, H, seed, hstd)
    W = synth.weight(V, H, seed, wstd)
    y = synth.labels(T, V, seed)
    return h, W, y


# --------------------------------------------------------------------------------------------
# fp64 oracle vs the scalar fsum oracle (independent implementations)
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,H,V", [(5, 24, 7), (3, 40, 1), (4, 8, 2), (6, 16, 11)])
def test_fp64_matches_brute_forward(T, H, V):
    h, W, y = _rand_case(T, H, V, seed=3)
    y = y.clone()
    if T >= 4:
        y[1] = -1      # out of range: logprob 0
        y[2] = V       # out of range
    ref_lp, ref_ent, ref_lse = brute.forward(h, W, y)
    out = fp64.forward(h, W, y)
    np.testing.assert_allclose(out["logprob"], ref_lp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["entropy"], ref_ent, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["lse"], ref_lse, rtol=0, atol=1e-12)
    if T >= 4:
        assert out["logprob"][1] == 0.0 and out["logprob"][2] == 0.0


def test_fp64_matches_brute_nonsquare_transposes():
    # H != V != T so that any transposed operand changes shapes or values.
    h, W, y = _rand_case(3, 10, 6, seed=11)
    lp, ent, lse = brute.forward(h, W, y)
    out = fp64.forward(h, W, y)
    np.testing.assert_allclose(out["logprob"], lp, atol=1e-12, rtol=0)
    np.testing.assert_allclose(out["entropy"], ent, atol=1e-12, rtol=0)


@pytest.mark.parametrize("T,H,V", [(4, 12, 5), (3, 8, 9)])
def test_fp64_matches_brute_backward(T, H, V):
    h, W, y = _rand_case(T, H, V, seed=5)
    y = y.clone()
    y[0] = -100        # out-of-range label: no onehot term
    g = synth.upstream_grad(T, 5)
    gh_ref, gW_ref = brute.backward(h, W, y, g)
    gh, gW = fp64.backward(h, W, y, g)
    np.testing.assert_allclose(gh, gh_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(gW, gW_ref, atol=1e-12, rtol=0)
    # sampled-row helpers agree with the full backward
    np.testing.assert_allclose(fp64.grad_hidden_rows(h, W, y, g, [2, 0]), gh[[2, 0]], atol=1e-13, rtol=0)
    np.testing.assert_allclose(fp64.grad_weight_rows(h, W, y, g, [V - 1, 1]), gW[[V - 1, 1]], atol=1e-13, rtol=0)


# --------------------------------------------------------------------------------------------
# closed forms and invariants of the log-softmax / gather
# --------------------------------------------------------------------------------------------

def test_probabilities_sum_to_one_and_lse_identical():
    V, H = 13, 32
    h1, W, _ = _rand_case(1, H, V, seed=7)
    h = h1.repeat(V, 1)
    y = torch.arange(V, dtype=torch.int32)
    out = fp64.forward(h, W, y)
    assert abs(math.fsum(np.exp(out["logprob"])) - 1.0) < 1e-12
    assert np.all(out["lse"] == out["lse"][0])
    assert np.all(out["entropy"] == out["entropy"][0])
    # gather index: logprob at label j equals z_j - lse
    z = fp64.to_f64(h1) @ fp64.to_f64(W).T
    np.testing.assert_allclose(out["logprob"], z[0] - out["lse"][0], atol=1e-13, rtol=0)


@pytest.mark.parametrize("V,expected", [(4096, -8.317766166719343), (152064, -11.932056763842207)])
def test_uniform_logits_give_minus_log_v(V, expected):
    # ln 4096 = 12 ln 2; ln 152064 = 8 ln 2 + ln 594 (594 = 2 * 3^3 * 11).
    assert abs(expected + (8 * math.log(2) + math.log(594) if V == 152064 else 12 * math.log(2))) < 1e-12
    H = 8
    h = torch.zeros((3, H), dtype=torch.bfloat16)          # h = 0 -> all logits 0
    W = synth.weight(V, H, 1, 0.02)
    y = torch.tensor([0, V // 2, V - 1], dtype=torch.int32)
    out = fp64.forward(h, W, y)
    np.testing.assert_allclose(out["logprob"], expected, atol=1e-12, rtol=0)
    np.testing.assert_allclose(out["entropy"], -expected, atol=1e-12, rtol=0)
    # W = 0 gives the same
    out2 = fp64.forward(synth.hidden(3, H, 2), torch.zeros((V, H), dtype=torch.bfloat16), y)
    np.testing.assert_allclose(out2["logprob"], expected, atol=1e-12, rtol=0)


def test_single_vocab_entry():
    h, W, _ = _rand_case(4, 16, 1, seed=9)
    out = fp64.forward(h, W, torch.zeros(4, dtype=torch.int32))
    assert np.all(out["logprob"] == 0.0)
    assert np.all(np.abs(out["entropy"]) <= 1e-15)


def test_two_vocab_entries_softplus():
    # bf16-exact integers: z = h @ W^T is known by hand.
    h = _bf16([[1.0, 2.0], [3.0, -1.0], [0.5, 0.25]])
    W = _bf16([[3.0, 0.0], [0.0, 1.0]])
    z = [[3.0, 2.0], [9.0, -1.0], [1.5, 0.25]]
    y = torch.tensor([0, 1, 1], dtype=torch.int32)
    out = fp64.forward(h, W, y)
    for t in range(3):
        zy, zo = z[t][y[t]], z[t][1 - y[t]]
        lp = -math.log1p(math.exp(zo - zy))
        p = 1.0 / (1.0 + math.exp(z[t][1] - z[t][0]))
        ent = -(p * math.log(p) + (1 - p) * math.log1p(-p))
        assert abs(out["logprob"][t] - lp) < 1e-13
        assert abs(out["entropy"][t] - ent) < 1e-13


def test_shift_invariance():
    T, H, V, c = 6, 32, 50, 8.0
    h, W, y = _rand_case(T, H, V, seed=13)
    h2 = torch.cat([h, torch.ones((T, 1), dtype=torch.bfloat16)], dim=1)
    W2 = torch.cat([W, torch.full((V, 1), c, dtype=torch.bfloat16)], dim=1)
    a = fp64.forward(h, W, y)
    b = fp64.forward(h2, W2, y)
    np.testing.assert_allclose(b["logprob"], a["logprob"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(b["entropy"], a["entropy"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(b["lse"], a["lse"] + c, atol=1e-12, rtol=0)


def test_one_hot_design_exact_logits():
    V = H = 16
    a = 3.5
    W = torch.eye(V, dtype=torch.bfloat16)
    ks = [0, 5, 15, 7]
    h = torch.zeros((len(ks), H), dtype=torch.bfloat16)
    for t, k in enumerate(ks):
        h[t, k] = a
    y = torch.tensor([0, 6, 15, 3], dtype=torch.int32)
    out = fp64.forward(h, W, y)
    S = math.exp(a) + V - 1
    for t, k in enumerate(ks):
        lp = (a if int(y[t]) == k else 0.0) - math.log(S)
        ent = math.log(S) - a * math.exp(a) / S
        assert abs(out["logprob"][t] - lp) < 1e-13
        assert abs(out["entropy"][t] - ent) < 1e-13


@pytest.mark.parametrize("delta", [5.0, 12.0, 20.0])
def test_peaked_row_entropy_closed_form(delta):
    # one logit at delta, V-1 logits at 0:  eps = (V-1) e^-delta,
    # H = log1p(eps) + delta * eps / (1 + eps)   (a rearrangement that is exact and stable).
    V = 16
    W = torch.eye(V, dtype=torch.bfloat16)
    h = torch.zeros((1, V), dtype=torch.bfloat16)
    h[0, 3] = delta
    out = fp64.forward(h, W, torch.tensor([3], dtype=torch.int32))
    eps = (V - 1) * math.exp(-delta)
    ent = math.log1p(eps) + delta * eps / (1 + eps)
    assert abs(out["entropy"][0] - ent) <= 1e-6 * ent
    assert abs(out["logprob"][0] + math.log1p(eps)) <= 1e-6 * math.log1p(eps)


# --------------------------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------------------------

def _objective(h, W, y, g):
    """sum_t g_t * logprob_t for in-range labels, and the gradient convention's objective
    -g_t * lse_t for out-of-range labels (their backward keeps only the -softmax term)."""
    out = fp64.forward(h, W, y)
    V = W.shape[0]
    valid = (y >= 0) & (y < V)
    return float(np.sum(np.where(valid, g * out["logprob"], -g * out["lse"])))


def test_backward_matches_central_differences():
    T, H, V = 3, 5, 4
    rng = np.random.default_rng(0)
    h = rng.normal(size=(T, H))
    W = rng.normal(size=(V, H)) * 0.7
    y = np.array([1, -1, 3])
    g = rng.normal(size=T)
    gh, gW = fp64.backward(h, W, y, g)
    eps = 1e-6
    for arr, grad in ((h, gh), (W, gW)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            fp = _objective(h, W, y, g)
            arr[idx] = old - eps
            fm = _objective(h, W, y, g)
            arr[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_backward_zero_hidden_closed_form():
    T, H, V = 4, 6, 9
    W = synth.weight(V, H, 3, 0.5)
    h = torch.zeros((T, H), dtype=torch.bfloat16)
    y = synth.labels(T, V, 3)
    g = synth.upstream_grad(T, 3)
    gh, gW = fp64.backward(h, W, y, g)
    assert np.all(gW == 0.0)
    Wf = fp64.to_f64(W)
    expect = fp64.to_f64(g)[:, None] * (Wf[y.long().numpy()] - Wf.mean(axis=0)[None, :])
    np.testing.assert_allclose(gh, expect, atol=1e-13, rtol=0)


def test_grad_weight_column_sums():
    T, H, V = 7, 12, 10
    h, W, y = _rand_case(T, H, V, seed=17)
    y = y.clone()
    y[3] = V + 4   # out of range
    g = synth.upstream_grad(T, 17)
    _, gW = fp64.backward(h, W, y, g)
    # rows of dz sum to 0 except for out-of-range labels, whose rows sum to -g_t
    hf, gf = fp64.to_f64(h), fp64.to_f64(g)
    expect = -gf[3] * hf[3]
    np.testing.assert_allclose(gW.sum(axis=0), expect, atol=1e-12, rtol=0)


@pytest.mark.parametrize("tau,with_ge", [(1.0, False), (0.8, True)])
def test_backward_shards_add_up_to_the_whole(tau, with_ge):
    # Linearity: the shares of a partition of the vocabulary sum to the whole backward, and the
    # grad_weight rows are the whole backward's rows (labels in every shard, one out of range).
    T, H, V = 9, 10, 11
    h, W, y = _rand_case(T, H, V, seed=41)
    y = y.clone()
    y[:4] = torch.tensor([0, 4, 8, 10], dtype=y.dtype)
    y[4] = -100
    g = synth.upstream_grad(T, 41)
    ge = synth.upstream_grad(T, 42) if with_ge else None
    gh, gW = fp64.backward(h, W, y, g, temperature=tau, grad_entropy=ge)
    bounds = [0, 3, 4, 8, V]
    shares = [fp64.backward_shard(h, W, y, g, a, b, temperature=tau, grad_entropy=ge)
              for a, b in zip(bounds[:-1], bounds[1:])]
    np.testing.assert_allclose(sum(s[0] for s in shares), gh, rtol=0, atol=1e-12 * np.abs(gh).max())
    np.testing.assert_allclose(np.concatenate([s[1] for s in shares]), gW, rtol=0, atol=1e-12 * np.abs(gW).max())
    # a shard without any of the labels has no label term: its share is -g sum_v p_v W_v (tau = 1,
    # no entropy gradient), checked against the brute-force probabilities
    if not with_ge:
        yb = y.clone()
        yb[:] = 0
        gh1, _ = fp64.backward_shard(h, W, yb, g, 5, V)
        z = fp64.to_f64(h) @ fp64.to_f64(W).T
        p = np.exp(z - z.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        expect = -fp64.to_f64(g)[:, None] * (p[:, 5:] @ fp64.to_f64(W)[5:])
        np.testing.assert_allclose(gh1, expect, rtol=0, atol=1e-12 * np.abs(expect).max())


# --------------------------------------------------------------------------------------------
# temperature, sum of squared probabilities, entropy gradient
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,H,V,tau", [(4, 24, 7, 0.7), (3, 16, 5, 1.7), (2, 8, 1, 0.25)])
def test_fp64_matches_brute_with_temperature(T, H, V, tau):
    h, W, y = _rand_case(T, H, V, seed=21)
    ref = fp64.forward(h, W, y, temperature=tau, sum_p2=True)
    lp, ent, lse = brute.forward(h, W, y, temperature=tau)
    p2 = brute.sum_p2(h, W, temperature=tau)
    np.testing.assert_allclose(ref["logprob"], lp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["entropy"], ent, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["lse"], lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["sum_p2"], p2, rtol=0, atol=1e-12)


def test_fp64_matches_brute_backward_temperature_and_entropy_grad():
    T, H, V = 4, 12, 5
    h, W, y = _rand_case(T, H, V, seed=22)
    y = y.clone()
    y[2] = -100
    g = synth.upstream_grad(T, 22)
    ge = synth.upstream_grad(T, 23)
    for tau, gE in ((0.6, None), (1.0, ge), (1.3, ge)):
        gh, gW = fp64.backward(h, W, y, g, temperature=tau, grad_entropy=gE)
        bgh, bgW = brute.backward(h, W, y, g, temperature=tau, grad_entropy=gE)
        np.testing.assert_allclose(gh, np.array(bgh), rtol=0, atol=1e-12)
        np.testing.assert_allclose(gW, np.array(bgW), rtol=0, atol=1e-12)


@pytest.mark.parametrize("tau", [0.5, 1.0, 2.5])
def test_one_hot_design_with_temperature(tau):
    # z_k = a at the hot index, 0 elsewhere, so z / tau is known exactly
    V = H = 16
    a = 3.5
    W = torch.eye(V, dtype=torch.bfloat16)
    ks = [0, 5, 15, 7]
    h = torch.zeros((len(ks), H), dtype=torch.bfloat16)
    for t, k in enumerate(ks):
        h[t, k] = a
    y = torch.tensor([0, 6, 15, 3], dtype=torch.int32)
    out = fp64.forward(h, W, y, temperature=tau, sum_p2=True)
    b = a / tau
    S = math.exp(b) + V - 1
    for t, k in enumerate(ks):
        lp = (b if int(y[t]) == k else 0.0) - math.log(S)
        ent = math.log(S) - b * math.exp(b) / S
        p2 = (math.exp(2 * b) + V - 1) / S ** 2
        assert abs(out["logprob"][t] - lp) < 1e-13
        assert abs(out["entropy"][t] - ent) < 1e-13
        assert abs(out["sum_p2"][t] - p2) < 1e-14
        assert abs(out["lse"][t] - math.log(S)) < 1e-13


def test_two_vocab_entries_softplus_with_temperature():
    tau = 0.37
    h, W, y = _rand_case(6, 8, 2, seed=24)
    out = fp64.forward(h, W, y, temperature=tau, sum_p2=True)
    z = fp64.to_f64(h) @ fp64.to_f64(W).T / tau
    for t in range(6):
        k = int(y[t])
        d = z[t, 1 - k] - z[t, k]
        lp = -(max(d, 0.0) + math.log1p(math.exp(-abs(d))))       # -softplus(d)
        p = math.exp(lp)
        assert abs(out["logprob"][t] - lp) < 1e-12
        assert abs(out["sum_p2"][t] - (p * p + (1 - p) ** 2)) < 1e-12


def test_high_temperature_limit_is_uniform():
    V = 4096
    h, W, y = _rand_case(3, 32, V, seed=25)
    out = fp64.forward(h, W, y, temperature=1e12, sum_p2=True)   # |z| / tau ~ 1e-11
    np.testing.assert_allclose(out["entropy"], math.log(V), rtol=0, atol=1e-9)
    np.testing.assert_allclose(out["logprob"], -math.log(V), rtol=0, atol=1e-9)
    np.testing.assert_allclose(out["sum_p2"], 1.0 / V, rtol=1e-9, atol=0)


def test_sum_p2_uniform_and_single_entry():
    out = fp64.forward(torch.zeros((2, 8), dtype=torch.bfloat16), synth.weight(1000, 8, 1, 1.0),
                       torch.tensor([3, 999], dtype=torch.int32), sum_p2=True)
    np.testing.assert_allclose(out["sum_p2"], 1e-3, rtol=1e-13, atol=0)
    h, W, y = _rand_case(3, 8, 1, seed=26)
    np.testing.assert_allclose(fp64.forward(h, W, y, sum_p2=True)["sum_p2"], 1.0, rtol=0, atol=1e-15)


def _objective_full(h, W, y, g, tau, ge):
    """sum_t g_t * (logprob_t, or -lse_t for an out-of-range label) + sum_t ge_t * entropy_t."""
    out = fp64.forward(h, W, y, temperature=tau)
    V = W.shape[0]
    valid = (y >= 0) & (y < V)
    f = np.sum(np.where(valid, g * out["logprob"], -g * out["lse"]))
    if ge is not None:
        f += np.sum(ge * out["entropy"])
    return float(f)


@pytest.mark.parametrize("tau,with_entropy", [(0.6, False), (1.0, True), (2.2, True)])
def test_backward_with_temperature_and_entropy_matches_central_differences(tau, with_entropy):
    T, H, V = 3, 5, 4
    rng = np.random.default_rng(1)
    h = rng.normal(size=(T, H))
    W = rng.normal(size=(V, H)) * 0.7
    y = np.array([1, -1, 3])
    g = rng.normal(size=T)
    ge = rng.normal(size=T) if with_entropy else None
    gh, gW = fp64.backward(h, W, y, g, temperature=tau, grad_entropy=ge)
    eps = 1e-6
    for arr, grad in ((h, gh), (W, gW)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            fp = _objective_full(h, W, y, g, tau, ge)
            arr[idx] = old - eps
            fm = _objective_full(h, W, y, g, tau, ge)
            arr[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def _golden_temperatures():
    rows = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "bf16_temperatures.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                t, b = line.split()
                rows.append((float(t), float(b)))
    return rows


def test_bf16_rounded_temperatures_printed_on_the_pages():
    rows = _golden_temperatures()
    assert len(rows) == 3
    for t, b in rows:
        assert torch.tensor(t, dtype=torch.float32).to(torch.bfloat16).item() == b
    # the rounded temperature is a different input: on a random case it moves log-probs by more
    # than the 2e-3 gate, so a path that rounded the temperature to bf16 would fail parity
    h, W, y = _rand_case(64, 64, 512, seed=27, wstd=0.6)
    for t, b in rows:
        d = fp64.forward(h, W, y, temperature=float(np.float32(t)))["logprob"] - \
            fp64.forward(h, W, y, temperature=b)["logprob"]
        assert np.abs(d).max() > 2e-3
