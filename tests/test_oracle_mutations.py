"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one.

Each mutant replaces one internal step of ``oracle.fp64`` via monkeypatch; the pins in
``test_oracle_pins`` are then run against the mutant and at least one must fail.
"""
import numpy as np
import pytest
import torch

from oracle import fp64
from tests import test_oracle_pins as pins


def _terms_transposed_shift(hb, W, tau=1.0):
    z = hb @ W.T / tau
    M = z.max(axis=1)
    S = np.exp(z - M[:, None]).sum(axis=1)
    lse = M + np.log(S)
    return z, lse, z - lse[:, None] + 1e-3        # off by a constant


def _terms_no_max(hb, W, tau=1.0):
    z = hb @ W.T / tau
    M = z.max(axis=1)
    S = np.exp(z - M[:, None]).sum(axis=1)
    lse = np.log(S)                                # dropped the max term
    return z, lse, z - lse[:, None]


def _gather_next(logp, yb, V):
    out = np.zeros(logp.shape[0])
    valid = (yb >= 0) & (yb < V)
    r = np.nonzero(valid)[0]
    out[r] = logp[r, (yb[r] + 1) % V]              # wrong index
    return out


def _dz_sign(logp, yb, gb, V, tau=1.0, ge=None):
    dz = np.exp(logp) * gb[:, None]                # wrong sign of the softmax term
    valid = (yb >= 0) & (yb < V)
    r = np.nonzero(valid)[0]
    dz[r, yb[r]] += gb[r]
    return dz / tau


def _dz_no_onehot(logp, yb, gb, V, tau=1.0, ge=None):
    return -np.exp(logp) * gb[:, None] / tau       # dropped the label term


def _terms_times_tau(hb, W, tau=1.0):
    z = hb @ W.T * tau                             # multiplied instead of divided
    M = z.max(axis=1)
    S = np.exp(z - M[:, None]).sum(axis=1)
    lse = M + np.log(S)
    return z, lse, z - lse[:, None]


_dz_right = fp64._dz_block


def _dz_no_tau(logp, yb, gb, V, tau=1.0, ge=None):
    return _dz_right(logp, yb, gb, V, 1.0, ge)     # dropped the 1/tau chain-rule factor


def _dz_entropy_sign(logp, yb, gb, V, tau=1.0, ge=None):
    return _dz_right(logp, yb, gb, V, tau, None if ge is None else -ge)   # wrong sign


def _dz_entropy_no_h(logp, yb, gb, V, tau=1.0, ge=None):
    p = np.exp(logp)
    dz = -p * gb[:, None]
    valid = (yb >= 0) & (yb < V)
    r = np.nonzero(valid)[0]
    dz[r, yb[r]] += gb[r]
    if ge is not None:
        dz -= ge[:, None] * p * logp               # dropped the + entropy term
    return dz / tau


def _sum_p_not_squared(p):
    return p.sum(axis=1)


_shard_right = fp64.backward_shard


def _shard_local_softmax(hidden, weight, labels, grad, v0, v1, row_block=128, temperature=1.0, grad_entropy=None):
    # the softmax taken over the shard's own rows instead of the whole vocabulary
    y = fp64._labels(labels) - v0
    y[(y < 0) | (y >= v1 - v0)] = -1
    gh, gw = fp64.backward(hidden, weight[v0:v1], torch.as_tensor(y), grad, row_block, temperature, grad_entropy)
    return gh, gw


def _shard_label_everywhere(hidden, weight, labels, grad, v0, v1, row_block=128, temperature=1.0, grad_entropy=None):
    # every shard adds the label term (it belongs to the owner only)
    gh, gw = _shard_right(hidden, weight, labels, grad, v0, v1, row_block, temperature, grad_entropy)
    y = fp64._labels(labels)
    W = fp64.to_f64(weight)
    g = fp64.to_f64(grad)
    r = np.nonzero((y >= 0) & (y < W.shape[0]) & ((y < v0) | (y >= v1)))[0]
    gh[r] += (g[r] / float(temperature))[:, None] * W[y[r]]
    return gh, gw


PIN_SETS = {
    "forward": [
        lambda: pins.test_fp64_matches_brute_forward(5, 24, 7),
        pins.test_probabilities_sum_to_one_and_lse_identical,
        lambda: pins.test_uniform_logits_give_minus_log_v(4096, -8.317766166719343),
        pins.test_two_vocab_entries_softplus,
        pins.test_one_hot_design_exact_logits,
    ],
    "backward": [
        lambda: pins.test_fp64_matches_brute_backward(4, 12, 5),
        pins.test_backward_matches_central_differences,
        pins.test_backward_zero_hidden_closed_form,
        pins.test_grad_weight_column_sums,
    ],
    "temperature": [
        lambda: pins.test_fp64_matches_brute_with_temperature(4, 24, 7, 0.7),
        lambda: pins.test_one_hot_design_with_temperature(0.5),
        pins.test_two_vocab_entries_softplus_with_temperature,
        pins.test_high_temperature_limit_is_uniform,
    ],
    "backward_ext": [
        pins.test_fp64_matches_brute_backward_temperature_and_entropy_grad,
        lambda: pins.test_backward_with_temperature_and_entropy_matches_central_differences(0.6, False),
        lambda: pins.test_backward_with_temperature_and_entropy_matches_central_differences(2.2, True),
    ],
    "shards": [
        lambda: pins.test_backward_shards_add_up_to_the_whole(1.0, False),
        lambda: pins.test_backward_shards_add_up_to_the_whole(0.8, True),
    ],
    "sum_p2": [
        lambda: pins.test_fp64_matches_brute_with_temperature(4, 24, 7, 0.7),
        lambda: pins.test_one_hot_design_with_temperature(1.0),
        pins.test_sum_p2_uniform_and_single_entry,
    ],
}


def _some_pin_fails(kind):
    for fn in PIN_SETS[kind]:
        try:
            fn()
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name,target,mutant,kind", [
    ("logp offset", "_block_softmax_terms", _terms_transposed_shift, "forward"),
    ("lse without max", "_block_softmax_terms", _terms_no_max, "forward"),
    ("gather wrong index", "_gather_label", _gather_next, "forward"),
    ("dz sign", "_dz_block", _dz_sign, "backward"),
    ("dz without onehot", "_dz_block", _dz_no_onehot, "backward"),
    ("temperature multiplies", "_block_softmax_terms", _terms_times_tau, "temperature"),
    ("dz without 1/tau", "_dz_block", _dz_no_tau, "backward_ext"),
    ("entropy gradient sign", "_dz_block", _dz_entropy_sign, "backward_ext"),
    ("entropy gradient without the entropy term", "_dz_block", _dz_entropy_no_h, "backward_ext"),
    ("sum_p2 not squared", "_sum_p2", _sum_p_not_squared, "sum_p2"),
    ("shard softmax over its own rows", "backward_shard", _shard_local_softmax, "shards"),
    ("label term in every shard", "backward_shard", _shard_label_everywhere, "shards"),
])
def test_pins_catch_planted_mistake(monkeypatch, name, target, mutant, kind):
    monkeypatch.setattr(fp64, target, mutant)
    assert _some_pin_fails(kind), f"no pin caught the planted mistake: {name}"


def test_unmutated_oracle_passes_all_pins():
    assert not any(_some_pin_fails(kind) for kind in PIN_SETS)
