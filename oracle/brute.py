"""Scalar brute-force oracle — TEST INFRASTRUCTURE ONLY, tiny shapes.

A second implementation of the same definition as ``oracle.fp64``, sharing no code with it:
pure-Python floats, every sum a correctly rounded ``math.fsum``, every ``exp``/``log`` a scalar
libm call.  bf16 x bf16 products are exact in a Python float, so each logit is the correctly
rounded exact dot product.  It exists to pin ``oracle.fp64`` (a transposed operand, a dropped
term or a wrong index in either one makes them disagree).

Definition followed (same passages as ``oracle.fp64``): log-prob = full-vocabulary log-softmax
gathered at the label, 0 for a label outside [0, V) (verl PR #8026 first review, sampler formula;
SkyRL PR #1765 precision-policy commit); entropy = -sum p log p of the same softmax; backward
dz = g * (onehot - p) with no onehot term out of range (SkyRL PR #1765 precision-policy and
streaming-backward commits).  With a temperature every logit is divided by it before the softmax
and the logit gradient carries 1/tau (verl PR #8026, review on the temperature order); the
optional companions are sum_j p_j^2 (verl PR #8026, first review: sum_pi_squared next to the
entropy) and the entropy's logit gradient -p_j (log p_j + entropy), which the pages leave
unwired (SkyRL PR #1765, PR summary).
"""
from __future__ import annotations

import math

import torch


def _rows(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).tolist()
    return [[float(v) for v in r] for r in x]


def _ints(y):
    if isinstance(y, torch.Tensor):
        return [int(v) for v in y.detach().to("cpu").to(torch.int64).tolist()]
    return [int(v) for v in y]


def _logits(h_row, W, tau=1.0):
    return [math.fsum(a * b for a, b in zip(h_row, w_row)) / tau for w_row in W]


def _lse(z):
    m = max(z)
    return m + math.log(math.fsum(math.exp(v - m) for v in z))


def forward(hidden, weight, labels, temperature=1.0):
    """Returns (logprob, entropy, lse) as Python lists of floats."""
    h, W, y = _rows(hidden), _rows(weight), _ints(labels)
    tau = float(temperature)
    V = len(W)
    lps, ents, lses = [], [], []
    for t, h_row in enumerate(h):
        z = _logits(h_row, W, tau)
        lse = _lse(z)
        logp = [v - lse for v in z]
        lps.append(logp[y[t]] if 0 <= y[t] < V else 0.0)
        ents.append(-math.fsum(math.exp(a) * a for a in logp))
        lses.append(lse)
    return lps, ents, lses


def sum_p2(hidden, weight, temperature=1.0):
    """sum_j p_tj^2 per row, as a list."""
    h, W = _rows(hidden), _rows(weight)
    tau = float(temperature)
    out = []
    for h_row in h:
        z = _logits(h_row, W, tau)
        lse = _lse(z)
        out.append(math.fsum(math.exp(2.0 * (v - lse)) for v in z))
    return out


def _floats(x):
    return [float(v) for v in (x.tolist() if isinstance(x, torch.Tensor) else x)]


def backward(hidden, weight, labels, grad, temperature=1.0, grad_entropy=None):
    """Returns (grad_hidden [T][H], grad_weight [V][H]) as nested lists."""
    h, W, y = _rows(hidden), _rows(weight), _ints(labels)
    g = _floats(grad)
    ge = None if grad_entropy is None else _floats(grad_entropy)
    tau = float(temperature)
    T, V, H = len(h), len(W), len(h[0]) if h else 0
    dz = []
    for t in range(T):
        z = _logits(h[t], W, tau)
        lse = _lse(z)
        logp = [v - lse for v in z]
        row = [-g[t] * math.exp(a) for a in logp]
        if 0 <= y[t] < V:
            row[y[t]] += g[t]
        if ge is not None:
            ent = -math.fsum(math.exp(a) * a for a in logp)
            row = [r - ge[t] * math.exp(a) * (a + ent) for r, a in zip(row, logp)]
        dz.append([r / tau for r in row])
    gh = [[math.fsum(dz[t][j] * W[j][k] for j in range(V)) for k in range(H)] for t in range(T)]
    gW = [[math.fsum(dz[t][j] * h[t][k] for t in range(T)) for k in range(H)] for j in range(V)]
    return gh, gW
