"""Seeded synthetic inputs for the fused LM-head log-prob.

This module is shared by the CPU oracle tests, the GPU tests and the benchmark.  It holds none of
the method's arithmetic: it only draws random numbers with seeded torch CPU generators, scales
them, and rounds them to bf16 (round-to-nearest-even, torch's own conversion).  The same bytes are
handed to the GPU library and to the oracle.

The trained checkpoints the pages measure on (a 4-layer Qwen3-Omni-30B-A3B thinker in verl PR
#8026's description, Qwen3.6-35B-A3B in SkyRL PR #1765's benchmark) are not available; Gaussian
tensors at the same hidden and vocabulary sizes stand in for them.

Streams: every tensor of a case draws from its own generator, seeded with ``16*seed + stream``:
hidden = 0, weight = 1, labels = 2, peaked-row permutation = 3, probe placement = 4,
upstream gradient of the log-probs = 5, upstream gradient of the entropies = 6.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

STREAM_HIDDEN = 0
STREAM_WEIGHT = 1
STREAM_LABELS = 2
STREAM_PEAK = 3
STREAM_PLACE = 4
STREAM_GRAD = 5
STREAM_GRAD_ENTROPY = 6


def generator(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(16 * int(seed) + int(stream))
    return g


def hidden(T: int, H: int, seed: int = 0, std: float = 1.0) -> torch.Tensor:
    """bf16 [T, H], N(0, std^2) drawn in fp32 then rounded to bf16."""
    x = torch.randn((T, H), generator=generator(seed, STREAM_HIDDEN), dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def weight(V: int, H: int, seed: int = 0, std: float = 0.02,
           peaked_frac: float = 0.0, peaked_scale: float = 10.0) -> torch.Tensor:
    """bf16 [V, H], N(0, std^2); a seeded floor(peaked_frac*V) rows are scaled by peaked_scale in
    fp32 before the bf16 rounding (this makes some softmax rows very peaked)."""
    w = torch.randn((V, H), generator=generator(seed, STREAM_WEIGHT), dtype=torch.float32)
    w.mul_(std)
    n_peak = int(peaked_frac * V)
    if n_peak > 0:
        rows = peaked_rows(V, seed, peaked_frac)
        w[rows] *= peaked_scale
    return w.to(torch.bfloat16)


def peaked_rows(V: int, seed: int = 0, peaked_frac: float = 0.01) -> torch.Tensor:
    n_peak = int(peaked_frac * V)
    perm = torch.randperm(V, generator=generator(seed, STREAM_PEAK))
    return perm[:n_peak].sort().values


def labels(T: int, V: int, seed: int = 0) -> torch.Tensor:
    """int32 [T], uniform in [0, V) (none out of range)."""
    return torch.randint(0, V, (T,), generator=generator(seed, STREAM_LABELS), dtype=torch.int64).to(torch.int32)


def upstream_grad(T: int, seed: int = 0) -> torch.Tensor:
    """fp32 [T], N(0, 1): the gradient arriving on logprob."""
    return torch.randn((T,), generator=generator(seed, STREAM_GRAD), dtype=torch.float32)


def entropy_grad(T: int, seed: int = 0) -> torch.Tensor:
    """fp32 [T], N(0, 1): the gradient arriving on the entropies."""
    return torch.randn((T,), generator=generator(seed, STREAM_GRAD_ENTROPY), dtype=torch.float32)


def shard_bounds(V: int, shards: int, chunk: int = 128):
    """[(start, end)] of `shards` vocabulary shards on `chunk`-row boundaries: every shard but the
    last has ceil(V / shards / chunk) chunks."""
    size = -(-V // (shards * chunk)) * chunk
    return [(min(V, k * size), min(V, (k + 1) * size)) for k in range(shards)]


def placement(n: int, T: int, seed: int = 0, salt: int = 0) -> torch.Tensor:
    """n distinct row positions in [0, T), seeded (used to embed probe rows in filler batches)."""
    g = generator(seed, STREAM_PLACE)
    if salt:
        g.manual_seed(16 * int(seed) + STREAM_PLACE + 1_000_003 * int(salt))
    return torch.randperm(T, generator=g)[:n]


@dataclasses.dataclass
class Workload:
    name: str
    T: int
    H: int
    V: int
    hidden_std: float = 1.0
    weight_std: float = 0.02
    peaked_frac: float = 0.0
    entropy: bool = True
    backward: bool = False
    temperature: float = 1.0      # logits divided by this fp32 value
    sum_p2: bool = False          # also sum_j p_j^2
    entropy_grad: bool = False    # backward also carries an upstream gradient on the entropies
    shards: int = 1               # > 1: the step is shard 0 of this many vocabulary shards, then the fold


# The workloads the measurements are quoted on (names say what they are).
WORKLOADS = {
    "fwd_T64_H256_V4096": Workload("fwd_T64_H256_V4096", 64, 256, 4096, entropy=False),
    "fwd_T2048_H4096_V152064": Workload("fwd_T2048_H4096_V152064", 2048, 4096, 152064),
    "fwd_T8192_H4096_V152064_peaked": Workload("fwd_T8192_H4096_V152064_peaked", 8192, 4096, 152064,
                                               peaked_frac=0.01),
    "fwd_T16_H5120_V152064": Workload("fwd_T16_H5120_V152064", 16, 5120, 152064),
    "fwd_T64_H5120_V152064": Workload("fwd_T64_H5120_V152064", 64, 5120, 152064),
    "fwd_T256_H5120_V152064": Workload("fwd_T256_H5120_V152064", 256, 5120, 152064),
    "fwdbwd_T4096_H5120_V152064": Workload("fwdbwd_T4096_H5120_V152064", 4096, 5120, 152064, backward=True),
    # the extended entry points at the same sizes
    "fwd_T8192_H4096_V152064_peaked_tau0.7_p2": Workload("fwd_T8192_H4096_V152064_peaked_tau0.7_p2", 8192, 4096,
                                                         152064, peaked_frac=0.01, temperature=0.7, sum_p2=True),
    "fwd_T8192_H4096_V152064_peaked_shard0of8": Workload("fwd_T8192_H4096_V152064_peaked_shard0of8", 8192, 4096,
                                                         152064, peaked_frac=0.01, shards=8),
    "fwdbwd_T4096_H5120_V152064_tau0.7_egrad": Workload("fwdbwd_T4096_H5120_V152064_tau0.7_egrad", 4096, 5120, 152064,
                                                        backward=True, temperature=0.7, entropy_grad=True),
}


@dataclasses.dataclass
class Inputs:
    hidden: torch.Tensor          # bf16 [T, H]
    weight: torch.Tensor          # bf16 [V, H]
    labels: torch.Tensor          # int32 [T]
    grad: Optional[torch.Tensor]  # fp32 [T] or None
    grad_entropy: Optional[torch.Tensor] = None  # fp32 [T] or None


def make_inputs(T: int, H: int, V: int, seed: int = 0, hidden_std: float = 1.0,
                weight_std: float = 0.02, peaked_frac: float = 0.0, with_grad: bool = False) -> Inputs:
    return Inputs(
        hidden=hidden(T, H, seed, hidden_std),
        weight=weight(V, H, seed, weight_std, peaked_frac),
        labels=labels(T, V, seed),
        grad=upstream_grad(T, seed) if with_grad else None,
    )


def make_workload(name: str, seed: int = 0) -> Inputs:
    w = WORKLOADS[name]
    x = make_inputs(w.T, w.H, w.V, seed, w.hidden_std, w.weight_std, w.peaked_frac, with_grad=w.backward)
    if w.entropy_grad:
        x.grad_entropy = entropy_grad(w.T, seed)
    return x
