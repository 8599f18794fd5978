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

Parity pins (tests/test_oracle_pins.py): agreement with the scalar ``math.fsum`` oracle in
``oracle.brute`` on tiny shapes; sum_j exp(logprob_j) = 1; uniform logits give -log V and log V;
V = 1 and V = 2 closed forms; shift invariance; a one-hot design with exactly known logits; the
peaked-row closed form of the entropy; central finite differences of the backward; the ``h = 0``
closed form of both gradients; the column sums of ``grad_weight``.  No function here is unpinned.
"""
from __future__ import annotations

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


def _block_softmax_terms(hb: np.ndarray, W: np.ndarray):
    """Full logits of a block of rows and their log-softmax: returns (z, lse, logp)."""
    z = hb @ W.T                                    # [rows, V]
    M = z.max(axis=1)
    S = np.exp(z - M[:, None]).sum(axis=1)
    lse = M + np.log(S)
    logp = z - lse[:, None]
    return z, lse, logp


def _gather_label(logp: np.ndarray, yb: np.ndarray, V: int) -> np.ndarray:
    valid = (yb >= 0) & (yb < V)
    out = np.zeros(logp.shape[0], dtype=np.float64)
    r = np.nonzero(valid)[0]
    out[r] = logp[r, yb[r]]
    return out


def forward_rows(hidden, weight, labels, rows=None, entropy: bool = True,
                 row_block: int = DEFAULT_ROW_BLOCK) -> dict:
    """Forward for the selected token rows (all rows if ``rows`` is None).

    Returns a dict of float64 arrays: ``logprob``, ``lse`` and (if asked) ``entropy``, indexed like
    ``rows``.
    """
    h = to_f64(hidden)
    W = to_f64(weight)
    y = _labels(labels)
    V = W.shape[0]
    if rows is None:
        rows = np.arange(h.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    n = rows.shape[0]
    lp = np.zeros(n)
    lse = np.zeros(n)
    ent = np.zeros(n) if entropy else None
    for s in range(0, n, row_block):
        rb = rows[s:s + row_block]
        _, lse_b, logp = _block_softmax_terms(h[rb], W)
        lse[s:s + len(rb)] = lse_b
        lp[s:s + len(rb)] = _gather_label(logp, y[rb], V)
        if entropy:
            p = np.exp(logp)
            ent[s:s + len(rb)] = -(p * logp).sum(axis=1)
    out = {"logprob": lp, "lse": lse}
    if entropy:
        out["entropy"] = ent
    return out


def forward(hidden, weight, labels, entropy: bool = True, row_block: int = DEFAULT_ROW_BLOCK) -> dict:
    """Forward over every row: ``logprob[T]``, ``lse[T]``, ``entropy[T]`` (float64)."""
    return forward_rows(hidden, weight, labels, None, entropy, row_block)


def _dz_block(logp: np.ndarray, yb: np.ndarray, gb: np.ndarray, V: int) -> np.ndarray:
    """dz = g * (onehot(y) - p); the onehot term is absent for labels outside [0, V)."""
    dz = -np.exp(logp) * gb[:, None]
    valid = (yb >= 0) & (yb < V)
    r = np.nonzero(valid)[0]
    dz[r, yb[r]] += gb[r]
    return dz


def backward(hidden, weight, labels, grad, row_block: int = DEFAULT_ROW_BLOCK):
    """Gradients of ``sum_t grad_t * logprob_t``: returns (grad_hidden [T,H], grad_weight [V,H])."""
    h = to_f64(hidden)
    W = to_f64(weight)
    y = _labels(labels)
    g = to_f64(grad)
    T, V = h.shape[0], W.shape[0]
    gh = np.zeros_like(h)
    gW = np.zeros_like(W)
    for s in range(0, T, row_block):
        sl = slice(s, min(T, s + row_block))
        _, _, logp = _block_softmax_terms(h[sl], W)
        dz = _dz_block(logp, y[sl], g[sl], V)
        gh[sl] = dz @ W
        gW += dz.T @ h[sl]
    return gh, gW


def grad_hidden_rows(hidden, weight, labels, grad, rows, row_block: int = DEFAULT_ROW_BLOCK) -> np.ndarray:
    """grad_hidden for the selected token rows only (each row needs only its own logits)."""
    h = to_f64(hidden)
    W = to_f64(weight)
    y = _labels(labels)
    g = to_f64(grad)
    V = W.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], h.shape[1]))
    for s in range(0, rows.shape[0], row_block):
        rb = rows[s:s + row_block]
        _, _, logp = _block_softmax_terms(h[rb], W)
        out[s:s + len(rb)] = _dz_block(logp, y[rb], g[rb], V) @ W
    return out


def grad_weight_rows(hidden, weight, labels, grad, vocab_rows, row_block: int = DEFAULT_ROW_BLOCK) -> np.ndarray:
    """grad_weight for the selected vocabulary rows.  Every token's log-sum-exp is needed, so this
    makes one full pass over the logits."""
    h = to_f64(hidden)
    W = to_f64(weight)
    y = _labels(labels)
    g = to_f64(grad)
    T, V = h.shape[0], W.shape[0]
    vr = np.asarray(vocab_rows, dtype=np.int64)
    out = np.zeros((vr.shape[0], h.shape[1]))
    for s in range(0, T, row_block):
        sl = slice(s, min(T, s + row_block))
        _, _, logp = _block_softmax_terms(h[sl], W)
        dz = _dz_block(logp, y[sl], g[sl], V)
        out += dz[:, vr].T @ h[sl]
    return out
