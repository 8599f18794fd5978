"""The softmax term of the backward, pinned on its own.

For a label inside the vocabulary dz = g (onehot - p); in the whole-matrix gradient norm the label
term g_t h_t (grad_weight) or g_t W_y (grad_hidden) dominates, so a gate on the whole matrix hardly
sees the -g p part.  Here:
  * every label is out of range, so dz = -g p everywhere (SkyRL PR #1765 "[megatron] Triton
    backend for fused LM-head log-prob", precision-policy commit: out-of-vocab rows keep only the
    softmax term), and the 1e-2 gate binds the exp, the dz^T store and every vocabulary step;
  * grad_weight rows that hold no label are gated as a block and row by row;
  * the column sums of grad_weight are checked against their closed form (rows of dz sum to
    g (1[y in range] - 1)), which involves every entry of p of every token.
"""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from oracle import fp64
from tests.gpu_util import (GRAD_REL_FRO, assert_softmax_rows, column_sum_target, dev, label_rows, rel_fro,
                            to_dev)

pytestmark = pytest.mark.gpu


def _oov_labels(n: int, V: int) -> torch.Tensor:
    """n out-of-range labels, a mix of ignore ids, V and beyond, and the largest int32."""
    pool = [-100, -1, V, V + 7, 2**31 - 1]
    return torch.tensor([pool[i % len(pool)] for i in range(n)], dtype=torch.int32)


def _run(h, w, y, g):
    hd, wd, yd, gd = to_dev(h, w, y, g)
    _, _, lse = lmh.forward(hd, wd, yd, want_lse=True)
    gh, gw = lmh.backward(hd, wd, yd, gd, lse)
    torch.cuda.synchronize()
    return gh.cpu().double().numpy(), gw.cpu().double().numpy()


def _check_colsum(gw, h, y, g, V, what):
    tgt = column_sum_target(h, y, g, V)
    err = np.linalg.norm(gw.sum(axis=0) - tgt) / np.linalg.norm(tgt)
    print(f"{what} column sums: rel err {err:.3e} (target norm {np.linalg.norm(tgt):.3e})", flush=True)
    assert err <= GRAD_REL_FRO


# (40, 64, 140000): three 65536-row vocabulary steps, the last ragged; (300, 320, 4999) and
# (100, 192, 2053): large- and mid-T tiles with ragged T, H and V
@pytest.mark.parametrize("T,H,V", [(40, 64, 140000), (300, 320, 4999), (100, 192, 2053)])
def test_all_labels_out_of_range(T, H, V):
    print(f"[case] bwd all-oov T={T} H={H} V={V}", flush=True)
    x = synth.make_inputs(T, H, V, seed=T, weight_std=0.05, with_grad=True)
    y = _oov_labels(T, V)
    gh, gw = _run(x.hidden, x.weight, y, x.grad)
    rgh, rgw = fp64.backward(x.hidden, x.weight, y, x.grad)
    e1, e2 = rel_fro(gh, rgh), rel_fro(gw, rgw)
    print(f"rel fro grad_hidden {e1:.3e} grad_weight {e2:.3e}", flush=True)
    assert e1 <= GRAD_REL_FRO and e2 <= GRAD_REL_FRO
    assert_softmax_rows(gw, rgw, np.zeros(V, dtype=bool), f"all-oov {T}x{H}x{V}")
    _check_colsum(gw, x.hidden, y, x.grad, V, f"all-oov {T}x{H}x{V}")


# normal labels: whole-matrix gate plus the non-label rows on their own and the column sums
@pytest.mark.parametrize("T,H,V,n_oov", [(64, 128, 1000, 0), (40, 64, 140000, 2), (257, 256, 4099, 128)])
def test_softmax_rows_with_labels(T, H, V, n_oov):
    print(f"[case] bwd softmax rows T={T} H={H} V={V} oov={n_oov}", flush=True)
    x = synth.make_inputs(T, H, V, seed=T + 1, weight_std=0.05, with_grad=True)
    y = x.labels.clone()
    y[:n_oov] = _oov_labels(n_oov, V)
    gh, gw = _run(x.hidden, x.weight, y, x.grad)
    rgh, rgw = fp64.backward(x.hidden, x.weight, y, x.grad)
    assert rel_fro(gh, rgh) <= GRAD_REL_FRO and rel_fro(gw, rgw) <= GRAD_REL_FRO
    assert_softmax_rows(gw, rgw, label_rows(y.numpy(), V), f"{T}x{H}x{V}")
    if n_oov:
        _check_colsum(gw, x.hidden, y, x.grad, V, f"{T}x{H}x{V}")
    else:  # the column sums vanish; bounded against the scale sum_t |g_t| |h_t|
        scale = np.linalg.norm((np.abs(x.grad.double().numpy())[:, None] * np.abs(x.hidden.double().numpy())).sum(0))
        assert np.linalg.norm(gw.sum(axis=0)) <= 2e-3 * scale


def test_T4096_H5120_V152064_all_labels_out_of_range():
    """The forward+backward workload's inputs with every label out of range, in the launch
    configuration the benchmark times (all 4096 rows, three vocabulary steps): 16 sampled rows of
    each gradient against the oracle, and the column sums of the whole grad_weight against their
    closed form."""
    name = "fwdbwd_T4096_H5120_V152064"
    print(f"[case] {name} all labels out of range", flush=True)
    x = synth.make_workload(name)
    T, V = x.hidden.shape[0], x.weight.shape[0]
    y = _oov_labels(T, V)
    h, w, yd, g = to_dev(x.hidden, x.weight, y, x.grad)
    _, _, lse = lmh.forward(h, w, yd, want_lse=True)
    gh, gw = lmh.backward(h, w, yd, g, lse)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(7)
    trows = torch.randperm(T, generator=gen)[:16].numpy()
    vrows = torch.randperm(V, generator=gen)[:16].numpy()
    W64 = fp64.to_f64(x.weight)
    rgh = fp64.grad_hidden_rows(x.hidden, W64, y, x.grad, trows)
    e1 = rel_fro(gh.cpu().double().numpy()[trows], rgh)
    print(f"grad_hidden rel fro on 16 rows {e1:.3e}", flush=True)
    assert e1 <= GRAD_REL_FRO
    rgw = fp64.grad_weight_rows(x.hidden, W64, y, x.grad, vrows)
    assert_softmax_rows(gw.cpu().double().numpy()[vrows], rgw, np.zeros(16, dtype=bool), name)
    # every element of grad_weight enters the column sums
    colsum = gw.double().sum(dim=0).cpu().numpy()
    tgt = column_sum_target(x.hidden, y, x.grad, V)
    err = np.linalg.norm(colsum - tgt) / np.linalg.norm(tgt)
    print(f"column sums rel err {err:.3e}", flush=True)
    assert err <= GRAD_REL_FRO
