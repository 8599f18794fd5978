"""Calls on two streams at once, each with its own workspace: the library keeps no mutable state of
its own, so concurrent calls give the bits of the same calls made one after another."""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from tests.gpu_util import bits, dev, to_dev

pytestmark = pytest.mark.gpu


def _problem(T, H, V, seed):
    x = synth.make_inputs(T, H, V, seed=seed, weight_std=0.05, with_grad=True)
    h, w, y, g = to_dev(x.hidden, x.weight, x.labels, x.grad)
    f32 = dict(dtype=torch.float32, device=dev())
    out = dict(lp=torch.empty(T, **f32), ent=torch.empty(T, **f32), lse=torch.empty(T, **f32),
               gh=torch.empty((T, H), **f32), gw=torch.empty((V, H), **f32))
    ws = torch.empty(lmh.lmhead_logprob_fwd_workspace_size(T, H, V), dtype=torch.uint8, device=dev())
    wsb = torch.empty(lmh.lmhead_logprob_bwd_workspace_size(T, H, V), dtype=torch.uint8, device=dev())

    def run(stream):
        lmh.lmhead_logprob_fwd(h, w, y, out["lp"], out["ent"], out["lse"], ws, stream)
        lmh.lmhead_logprob_bwd(h, w, y, g, out["lse"], out["gh"], out["gw"], False, wsb, stream)

    return run, out


def test_two_streams_give_the_sequential_bits():
    # a large-T problem (persistent tiles), a small-T one (streaming tiles) and one whose forward
    # splits the tiles' K steps between workgroups (274 tiles)
    problems = [_problem(300, 256, 3000, 11), _problem(40, 192, 2053, 12), _problem(200, 264, 70000, 13)]
    cur = torch.cuda.current_stream()
    for run, _ in problems:
        run(cur)
    torch.cuda.synchronize()
    want = [{k: bits(v) for k, v in out.items()} for _, out in problems]

    streams = [torch.cuda.Stream() for _ in problems]
    for rep in range(3):
        for _, out in problems:
            for t in out.values():
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        for (run, _), s in zip(problems, streams):
            s.wait_stream(cur)
            run(s)
        torch.cuda.synchronize()
        for i, (_, out) in enumerate(problems):
            for k, v in out.items():
                assert np.array_equal(bits(v), want[i][k]), f"repeat {rep}: problem {i} {k} differs on two streams"
