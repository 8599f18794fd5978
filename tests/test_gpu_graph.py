"""The entry points under HIP graph capture: forward and backward recorded once, replayed several
times with the program's own eager work and synchronizations between replays, every replay bitwise
equal to the eager calls.  (The tile-counter resets inside the calls are kernels, not memsets.)"""
import numpy as np
import pytest
import torch

import lm_head_log_lmhead_amd as lmh
import synth
from tests.gpu_util import bits, dev, to_dev

pytestmark = pytest.mark.gpu


# streaming tiles, the dynamic large-T schedule, and the K-split schedule (274 vocabulary tiles,
# accumulators handed between workgroups, its counter and flags reset by a kernel in the call)
@pytest.mark.parametrize("T,H,V", [(40, 256, 3000), (300, 256, 3000), (200, 136, 70000)])
def test_forward_and_backward_replay_in_a_graph(T, H, V):
    print(f"[case] graph replay T={T} H={H} V={V}", flush=True)
    x = synth.make_inputs(T, H, V, seed=7, weight_std=0.05, with_grad=True)
    h, w, y, g = to_dev(x.hidden, x.weight, x.labels, x.grad)
    f32 = dict(dtype=torch.float32, device=dev())
    lp, ent, lse = (torch.empty(T, **f32) for _ in range(3))
    gh, gw = torch.empty((T, H), **f32), torch.empty((V, H), **f32)
    ws = torch.empty(lmh.lmhead_logprob_fwd_workspace_size(T, H, V), dtype=torch.uint8, device=dev())
    wsb = torch.empty(lmh.lmhead_logprob_bwd_workspace_size(T, H, V), dtype=torch.uint8, device=dev())

    def step():
        lmh.lmhead_logprob_fwd(h, w, y, lp, ent, lse, ws)
        lmh.lmhead_logprob_bwd(h, w, y, g, lse, gh, gw, False, wsb)

    step()
    torch.cuda.synchronize()
    want = [bits(t) for t in (lp, ent, lse, gh, gw)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (lp, ent, lse, gh, gw):
            t.fill_(float("nan"))                    # eager work between replays
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(t) for t in (lp, ent, lse, gh, gw)]
        for name, a, b in zip(("logprob", "entropy", "lse", "grad_hidden", "grad_weight"), got, want):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs from the eager call"
