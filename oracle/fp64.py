"""fp64 CPU oracle of the fused LM-head log-prob — TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may call this.  It is the plain
definition of what the fused path computes, written out with numpy float64 and no blocking,
fusion or reordering beyond splitting the token rows into independent blocks (every quantity is
per row, so row blocks change nothing).

What is computed, and where the pages define it:

* logits ``z = h @ W^T`` over the whole vocabulary.  The LM-head projection that the fused method
  folds into the log-prob (SkyRL PR #1765 "[megatron] Triton backend for fused LM-head log-prob",
  design commit: the vocab projection is folded into the chunked log-prob).  The inputs are bf16;
  every bf16 x bf16 product is exact in fp64, so ``z`` here is the exact logit up to fp64
  summation rounding (the pages keep fp32 logits; fp64 is the higher-precision reference).
* ``logprob_t = log_softmax(z_t)[y_t]``: a log-softmax over the full vocabulary, then a gather
  at the label (verl PR #8026 "batch-invariant actor forward and sampler log-prob formula",
  first review, the sampler log-prob formula hunk: fp32 log_softmax over the full vocab, then
  gather, float32 output whatever the logits dtype).  ``lse_t = M_t + log sum_j exp(z_tj - M_t)``.
* A label outside ``[0, V)`` yields logprob 0 (SkyRL PR #1765, precision-policy commit: the
  forward masks the out-of-vocab log-prob value to 0).
* ``entropy_t = -sum_j p_tj log p_tj`` with ``p = softmax(z_t)`` — the entropy of the same
  softmax, metric only, no gradient (verl PR #8026 first review: the entropy should be that of the
  fp32 log-softmax the log-probs come from; SkyRL PR #1765 maintainer review: entropy stays
  no-grad).  Natural log (nats).
* Backward of ``sum_t g_t * logprob_t``: ``dz_tj = g_t * ([j == y_t] - p_tj)``; for an
  out-of-range label the one-hot term is absent and ``dz = -g * p`` (SkyRL PR #1765,
  precision-policy commit: the backward passes grad_output through at out-of-vocab positions, so
  the -softmax term remains and the onehot term drops; streaming-backward commit: exp of the
  log-softmax, negate, multiply by the upstream gradient, then add it at the label).
  ``grad_hidden = dz @ W`` and ``grad_weight = dz^T @ h``.
* Temperature ``tau``: the logits are divided by it before the log-softmax, so every quantity
  above is that of ``softmax(z / tau)``, and the backward carries the chain-rule factor 1/tau.
  The division is of the full-precision logits by the caller's fp32 temperature, never by a
  bf16-rounded one (verl PR #8026, review on the temperature order: the sampler divides fp32
  logits by the fp32 temperature, and doing it on bf16 logits with a bf16 temperature changes
  every token).  Here the logits are fp64 and ``tau`` is the given value widened exactly.
* ``sum_p2_t = sum_j p_tj^2`` of the same softmax, a companion metric of the entropy that the
  pages compute from the same logits (verl PR #8026, first review and its follow-up: entropy and
  sum_pi_squared are kept next to the log-probs).
* Entropy gradient, which the pages leave unwired (SkyRL PR #1765, PR summary: entropy stays
  no-grad until its gradient is wired and validated): for ``sum_t gE_t * entropy_t`` the logit
  gradient is ``-gE_t * p_tj * (log p_tj + entropy_t)`` (with ``log p = z/tau - lse``), added to
  the log-prob term before the 1/tau factor.

Parity pins (tests/test_oracle_pins.py): agreement with the scalar ``math.fsum`` oracle in
``oracle.brute`` on tiny shapes; sum_j exp(logprob_j) = 1; uniform logits give -log V and log V;
V = 1 and V = 2 closed forms; shift invariance; a one-hot design with exactly known logits; the
peaked-row closed form of the entropy; central finite differences of the backward; the ``h = 0``
closed form of both gradients; the column sums of ``grad_weight``; with a temperature, the
one-hot, two-entry and infinite-temperature closed forms and finite differences; for
``sum_p2``, the one-hot and uniform closed forms; for the entropy gradient, finite differences of
the entropy; for a vocabulary shard's share of the backward, that the shares of a partition add
up to the whole backward.  No function here is unpinned.
"""
from __future__ import annotations

import math

import numpy as np
import torch

DEFAULT_ROW_BLOCK = 128


def to_f64(x) -> np.ndarray:
    """Exact widening of bf16 / fp32 tensors (or arrays) to float64 numpy arrays."""
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _labels(y) -> np.ndarray:
    if isinstance(y, torch.Tensor):
        return y.detach().to("cpu").to(torch.int64).numpy()
    return np.asarray(y, dtype=np.int64)


def _temperature(temperature) -> float:
    tau = float(temperature)
    if not (math.isfinite(tau) and tau > 0.0):
        raise ValueError(f"temperature must be finite and positive, got {temperature!r}")
    return tau


def _block_softmax_terms(hb: np.ndarray, W: np.ndarray, tau: float = 1.0):
    """Full logits of a block of rows, divided by the temperature, and their log-softmax:
    returns (z, lse, logp)."""
    z = (hb @ W.T) / tau                            # [rows, V]
    M = z.max(axis=1)
    S = np.exp(z - M[:, None]).sum(axis=1)
    lse = M + np.log(S)
    logp = z - lse[:, None]
    return z, lse, logp


def _sum_p2(p: np.ndarray) -> np.ndarray:
    return (p * p).sum(axis=1)


def _gather_label(logp: np.ndarray, yb: np.ndarray, V: int) -> np.ndarray:
    valid = (yb >= 0) & (yb < V)
    out = np.zeros(logp.shape[0], dtype=np.float64)
    r = np.nonzero(valid)[0]
    out[r] = logp[r, yb[r]]
    return out


def forward_rows(hidden, weight, labels, rows=None, entropy: bool = True,
                 row_block: int = DEFAULT_ROW_BLOCK, temperature=1.0, sum_p2: bool = False) -> dict:
    """Forward for the selected token rows (all rows if ``rows`` is None).

    Returns a dict of float64 arrays: ``logprob``, ``lse`` and, if asked, ``entropy`` and
    ``sum_p2``, indexed like ``rows``.  ``lse`` is that of the logits divided by the temperature.
    """
    h = to_f64(hidden)
    W = to_f64(weight)
    y = _labels(labels)
    tau = _temperature(temperature)
    V = W.shape[0]
    if rows is None:
        rows = np.arange(h.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    n = rows.shape[0]
    lp = np.zeros(n)
    lse = np.zeros(n)
    ent = np.zeros(n) if entropy else None
    p2 = np.zeros(n) if sum_p2 else None
    for s in range(0, n, row_block):
        rb = rows[s:s + row_block]
        _, lse_b, logp = _block_softmax_terms(h[rb], W, tau)
        lse[s:s + len(rb)] = lse_b
        lp[s:s + len(rb)] = _gather_label(logp, y[rb], V)
        if entropy or sum_p2:
            p = np.exp(logp)
        if entropy:
            ent[s:s + len(rb)] = -(p * logp).sum(axis=1)
        if sum_p2:
            p2[s:s + len(rb)] = _sum_p2(p)
    out = {"logprob": lp, "lse": lse}
    if entropy:
        out["entropy"] = ent
    if sum_p2:
        out["sum_p2"] = p2
    return out


def forward(hidden, weight, labels, entropy: bool = True, row_block: int = DEFAULT_ROW_BLOCK,
            temperature=1.0, sum_p2: bool = False) -> dict:
    """Forward over every row: ``logprob[T]``, ``lse[T]``, ``entropy[T]`` (and ``sum_p2[T]`` if
    asked), float64."""
    return forward_rows(hidden, weight, labels, None, entropy, row_block, temperature, sum_p2)


def _dz_block(logp: np.ndarray, yb: np.ndarray, gb: np.ndarray, V: int, tau: float = 1.0,
              ge: np.ndarray | None = None) -> np.ndarray:
    """Logit gradient of sum_t g_t logprob_t (+ sum_t ge_t entropy_t):
    (g * (onehot(y) - p) - ge * p * (log p + entropy)) / tau; the onehot term is absent for labels
    outside [0, V)."""
    p = np.exp(logp)
    dz = -p * gb[:, None]
    valid = (yb >= 0) & (yb < V)
    r = np.nonzero(valid)[0]
    dz[r, yb[r]] += gb[r]
    if ge is not None:
        ent = -(p * logp).sum(axis=1)
        dz -= ge[:, None] * p * (logp + ent[:, None])
    return dz / tau


def backward(hidden, weight, labels, grad, row_block: int = DEFAULT_ROW_BLOCK, temperature=1.0,
             grad_entropy=None):
    """Gradients of ``sum_t grad_t * logprob_t`` (+ ``sum_t grad_entropy_t * entropy_t``):
    returns (grad_hidden [T,H], grad_weight [V,H])."""
    h = to_f64(hidden)
    W = to_f64(weight)
    y = _labels(labels)
    g = to_f64(grad)
    ge = None if grad_entropy is None else to_f64(grad_entropy)
    tau = _temperature(temperature)
    T, V = h.shape[0], W.shape[0]
    gh = np.zeros_like(h)
    gW = np.zeros_like(W)
    for s in range(0, T, row_block):
        sl = slice(s, min(T, s + row_block))
        _, _, logp = _block_softmax_terms(h[sl], W, tau)
        dz = _dz_block(logp, y[sl], g[sl], V, tau, None if ge is None else ge[sl])
        gh[sl] = dz @ W
        gW += dz.T @ h[sl]
    return gh, gW


def backward_shard(hidden, weight, labels, grad, v0: int, v1: int, row_block: int = DEFAULT_ROW_BLOCK,
                   temperature=1.0, grad_entropy=None):
    """The share of the vocabulary rows [v0, v1) in the gradients, the softmax being over the
    whole vocabulary: returns (dz[:, v0:v1] @ W[v0:v1], grad_weight rows v0 .. v1-1).  The label
    term appears only in the shard that holds the label (SkyRL PR #1765, design commit: in the
    vocabulary-parallel path only the owner of a target contributes it).  By linearity the shares
    of a partition of the vocabulary add up to ``backward``."""
    h = to_f64(hidden)
    W = to_f64(weight)
    y = _labels(labels)
    g = to_f64(grad)
    ge = None if grad_entropy is None else to_f64(grad_entropy)
    tau = _temperature(temperature)
    T, V = h.shape[0], W.shape[0]
    if not 0 <= v0 <= v1 <= V:
        raise ValueError(f"shard [{v0}, {v1}) outside the vocabulary of {V}")
    gh = np.zeros_like(h)
    gW = np.zeros((v1 - v0, h.shape[1]))
    for s in range(0, T, row_block):
        sl = slice(s, min(T, s + row_block))
        _, _, logp = _block_softmax_terms(h[sl], W, tau)
        dz = _dz_block(logp, y[sl], g[sl], V, tau, None if ge is None else ge[sl])[:, v0:v1]
        gh[sl] = dz @ W[v0:v1]
        gW += dz.T @ h[sl]
    return gh, gW


def grad_hidden_rows(hidden, weight, labels, grad, rows, row_block: int = DEFAULT_ROW_BLOCK, temperature=1.0,
                     grad_entropy=None) -> np.ndarray:
    """grad_hidden for the selected token rows only (each row needs only its own logits)."""
    h = to_f64(hidden)
    W = to_f64(weight)
    y = _labels(labels)
    g = to_f64(grad)
    ge = None if grad_entropy is None else to_f64(grad_entropy)
    tau = _temperature(temperature)
    V = W.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], h.shape[1]))
    for s in range(0, rows.shape[0], row_block):
        rb = rows[s:s + row_block]
        _, _, logp = _block_softmax_terms(h[rb], W, tau)
        out[s:s + len(rb)] = _dz_block(logp, y[rb], g[rb], V, tau, None if ge is None else ge[rb]) @ W
    return out


def grad_weight_rows(hidden, weight, labels, grad, vocab_rows, row_block: int = DEFAULT_ROW_BLOCK,
                     temperature=1.0, grad_entropy=None) -> np.ndarray:
    """grad_weight for the selected vocabulary rows.  Every token's log-sum-exp is needed, so this
    makes one full pass over the logits."""
    h = to_f64(hidden)
    W = to_f64(weight)
    y = _labels(labels)
    g = to_f64(grad)
    ge = None if grad_entropy is None else to_f64(grad_entropy)
    tau = _temperature(temperature)
    T, V = h.shape[0], W.shape[0]
    vr = np.asarray(vocab_rows, dtype=np.int64)
    out = np.zeros((vr.shape[0], h.shape[1]))
    for s in range(0, T, row_block):
        sl = slice(s, min(T, s + row_block))
        _, _, logp = _block_softmax_terms(h[sl], W, tau)
        dz = _dz_block(logp, y[sl], g[sl], V, tau, None if ge is None else ge[sl])
        out += dz[:, vr].T @ h[sl]
    return out
