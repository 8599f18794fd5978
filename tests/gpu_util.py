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
