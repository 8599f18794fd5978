"""Helpers shared by the GPU tests: device transfer, calls through the C ABI, and the gates."""
import numpy as np
import torch

import lm_head_log_lmhead_amd as lmh

LOGPROB_ATOL = 2e-3          # |logprob - oracle| <= 2e-3
ENTROPY_RTOL = 1e-3          # |entropy - oracle| <= 1e-3 * |oracle| + 1e-7
ENTROPY_ATOL = 1e-7
GRAD_REL_FRO = 1e-2          # ||grad - oracle||_F <= 1e-2 * ||oracle||_F


def dev():
    return torch.device("cuda:0")


def to_dev(*ts):
    return [None if t is None else t.to(dev()) for t in ts]


def fwd(h, w, y, entropy=True):
    """Calls lmhead_logprob_fwd through the C ABI; returns float64 numpy arrays."""
    lp, ent, lse = lmh.forward(h, w, y, entropy=entropy, want_lse=True)
    torch.cuda.synchronize()
    return (lp.cpu().double().numpy(), None if ent is None else ent.cpu().double().numpy(),
            lse.cpu().double().numpy())


def fwd_raw(h, w, y):
    """Same call, fp32 tensors kept on the device (for bitwise comparisons)."""
    lp, ent, lse = lmh.forward(h, w, y, entropy=True, want_lse=True)
    torch.cuda.synchronize()
    return lp, ent, lse


def assert_logprob(got, want, what=""):
    err = np.abs(got - want)
    i = int(np.argmax(err)) if err.size else 0
    assert err.size == 0 or err.max() <= LOGPROB_ATOL, f"{what} logprob max err {err.max():.3e} at row {i}"


def assert_entropy(got, want, what=""):
    bound = ENTROPY_RTOL * np.abs(want) + ENTROPY_ATOL
    bad = np.abs(got - want) > bound
    assert not bad.any(), (f"{what} entropy: {int(bad.sum())} rows out of gate; first row {int(np.argmax(bad))}: "
                           f"got {got[np.argmax(bad)]!r} want {want[np.argmax(bad)]!r}")


def rel_fro(got, want):
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def label_rows(labels, V) -> np.ndarray:
    """Boolean [V]: vocabulary rows that hold the label of some token (their grad_weight row carries
    a label term g_t h_t besides the softmax term)."""
    y = np.asarray(labels, dtype=np.int64)
    mask = np.zeros(V, dtype=bool)
    mask[y[(y >= 0) & (y < V)]] = True
    return mask


def assert_softmax_rows(got, want, is_label, what=""):
    """grad_weight rows that hold no label carry only the softmax term -sum_t g_t p_tv h_t, which is
    a small share of the whole matrix's norm: they are gated on their own, as a block and row by
    row, so a wrong p cannot hide behind the label rows."""
    nl = ~np.asarray(is_label, dtype=bool)
    assert nl.any(), f"{what}: no non-label row to check"
    block = rel_fro(got[nl], want[nl])
    per_row = np.linalg.norm(got[nl] - want[nl], axis=1) / np.maximum(np.linalg.norm(want[nl], axis=1), 1e-300)
    worst = int(np.argmax(per_row))
    print(f"{what} non-label rows: {int(nl.sum())}, block rel fro {block:.3e}, worst row rel {per_row[worst]:.3e}",
          flush=True)
    assert block <= GRAD_REL_FRO, f"{what} non-label grad_weight rows: rel fro {block:.3e}"
    assert per_row[worst] <= GRAD_REL_FRO, f"{what} non-label grad_weight row {worst}: rel err {per_row[worst]:.3e}"


def column_sum_target(hidden, labels, grad, V) -> np.ndarray:
    """sum_v grad_weight[v, :] in closed form.  Each row of dz sums to g_t (1[y_t in range] - 1), so
    the column sums are -sum over out-of-range tokens of g_t h_t (fp64 from the exact inputs)."""
    h = hidden.detach().cpu().double().numpy()
    g = grad.detach().cpu().double().numpy()
    y = labels.detach().cpu().long().numpy()
    oov = (y < 0) | (y >= V)
    return -(g[oov, None] * h[oov]).sum(axis=0)
