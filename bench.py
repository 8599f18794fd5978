"""Benchmark of the fused LM-head log-prob on one MI355X.

Default workload: the forward (log-prob + entropy) at T=8192 tokens, H=4096, V=152064, bf16
inputs with the peaked-weight recipe (1% of weight rows x10), synthetic and seeded.

A step is one pass of the whole hot path over the batch, inputs resident in HBM: for forward
workloads lmhead_logprob_fwd, i.e. the logit-tile GEMM with its per-chunk records (stage 1) and
the fixed-order fold (stage 2); for the forward+backward workload also lmhead_logprob_bwd.
W warm-up steps, then K timed steps bracketed by torch.cuda.synchronize(); every stage launch is
also bracketed by HIP events on the stream the library launches on, which gives the dominant
kernel's average duration for the roofline.

``ms_per_step`` is the wall-clock mean over the K steps; ``ms_per_step_median`` the median of the
per-step durations from the events.  The CPU-baseline leg times the fp64 oracle on the first rows
of the same inputs, and ``parity`` compares the timed run's own outputs with the oracle's on those
rows (max |d logprob|, max relative entropy error, rows outside the gates).

Prints ONE JSON line.  ``--gpus N`` with N > 1 is not supported: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import lm_head_log_lmhead_amd as lmh  # noqa: E402
import synth  # noqa: E402

METRIC = "fused LM-head logprob tokens/s + % bf16 MFMA peak, T=8192 H=4096 V=152064"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
CSRC = os.path.join(ROOT, "lm_head_log_lmhead_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="fwd_T8192_H4096_V152064_peaked", choices=sorted(synth.WORKLOADS))
    p.add_argument("--cpu-sample-rows", type=int, default=-1,
                   help="rows of the workload the CPU oracle is timed on (0 disables the CPU baseline; "
                        "-1 sizes the sample to about CPU_TARGET_S seconds of oracle work)")
    p.add_argument("--bwd-workspace-mb", type=int, default=0,
                   help="run the backward with a workspace of this many MiB (0: the size of the fastest "
                        "schedule); the library then takes the widest vocabulary step that fits")
    p.add_argument("--fwd-workspace", choices=("fast", "min"), default="fast",
                   help="forward workspace: the size of the fastest schedule, or the smallest accepted "
                        "(no K-split accumulator slots: the dynamic whole-tile schedule everywhere)")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="also run a plain device copy of this many bytes (counter calibration)")
    return p.parse_args()


def kernel_sources_digest() -> str:
    """Digest of every source the library is built from (kernels, host code, the ABI header)."""
    h = hashlib.sha256()
    paths = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))] + [os.path.join(ROOT, "include",
                                                                                      "lmhead_logprob.h")]
    for path in paths:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter summary, if that
    summary was taken on the current kernel sources (else None)."""
    path = os.path.join(PROFILES, f"fwd_partials_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"sources digest:\s*`?([0-9a-f]{16})", text)
    t = re.search(r"traffic bytes per launch:\s*`?([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_sources_digest():
        return None
    return float(t.group(1))


CPU_TARGET_S = 15.0     # seconds of oracle work the automatic CPU sample aims at
CPU_PROBE_ROWS = 128    # rows timed first to size the automatic sample


LOGPROB_ATOL = 2e-3     # |logprob - oracle|
ENTROPY_RTOL = 1e-3     # |entropy - oracle| <= 1e-3 |oracle| + 1e-7
ENTROPY_ATOL = 1e-7


def parity(ref, lp, ent):
    """Errors of the timed run's outputs on the oracle's rows: max |d logprob|, max relative
    entropy error, and the number of rows outside either gate."""
    n = ref["logprob"].shape[0]
    d_lp = np.abs(lp[:n] - ref["logprob"])
    bad = d_lp > LOGPROB_ATOL
    out = {"rows": int(n), "max_abs_err_logprob": float(d_lp.max())}
    if ent is not None and "entropy" in ref:
        d_h = np.abs(ent[:n] - ref["entropy"])
        out["max_rel_err_entropy"] = float((d_h / np.maximum(np.abs(ref["entropy"]), 1e-300)).max())
        bad |= d_h > ENTROPY_RTOL * np.abs(ref["entropy"]) + ENTROPY_ATOL
    out["rows_outside_gates"] = int(bad.sum())
    return out


def cpu_baseline(x, rows: int, name: str, temperature: float = 1.0, sum_p2: bool = False):
    """Times the fp64 CPU oracle (as it stands) on the first `rows` rows of the same inputs; with
    rows < 0 the sample is sized from a short probe to about CPU_TARGET_S seconds (whole multiples
    of the probe, at most every row).  Returns the baseline and the oracle's outputs."""
    from oracle import fp64
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = os.cpu_count()
    T = x.hidden.shape[0]
    W = fp64.to_f64(x.weight)          # conversion is outside the timed region
    if rows < 0:
        probe = min(CPU_PROBE_ROWS, T)
        t0 = time.perf_counter()
        fp64.forward(x.hidden[:probe], W, x.labels[:probe], entropy=True, temperature=temperature, sum_p2=sum_p2)
        per_row = (time.perf_counter() - t0) / probe
        rows = int(min(T, max(probe, probe * round(CPU_TARGET_S / per_row / probe))))
    h = x.hidden[:rows]
    y = x.labels[:rows]
    t0 = time.perf_counter()
    ref = fp64.forward(h, W, y, entropy=True, temperature=temperature, sum_p2=sum_p2)
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {rows} of {x.hidden.shape[0]} rows of {name} (fp64 numpy, logprob+entropy), "
                      f"{dt:.1f} s"}, ref


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); multi-GPU sharding is not part of "
              "this build", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    wl = synth.WORKLOADS[a.workload]
    T, H, V = wl.T, wl.H, wl.V
    tau = float(np.float32(wl.temperature))
    dev = torch.device("cuda:0")
    print(f"[bench] generating {a.workload}", file=sys.stderr, flush=True)
    x = synth.make_workload(a.workload, seed=0)
    h, w, y = x.hidden.to(dev), x.weight.to(dev), x.labels.to(dev)
    lp = torch.empty(T, dtype=torch.float32, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev) if (wl.entropy or wl.entropy_grad) else None
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    p2 = torch.empty(T, dtype=torch.float32, device=dev) if wl.sum_p2 else None
    ws_size = (lmh.lmhead_logprob_fwd_workspace_size if a.fwd_workspace == "fast"
               else lmh.lmhead_logprob_fwd_workspace_size_min)
    ws = torch.empty(ws_size(T, H, V), dtype=torch.uint8, device=dev)
    # vocabulary shards: the step runs shard 0's partials, then the fold over every shard's records
    shards = synth.shard_bounds(V, wl.shards)
    v0, v1 = shards[0]
    Vp = v1 - v0                        # weight rows the partials stage computes per step
    if wl.backward:
        g = x.grad.to(dev)
        ge = x.grad_entropy.to(dev) if x.grad_entropy is not None else None
        gh = torch.empty((T, H), dtype=torch.float32, device=dev)
        gw = torch.empty((V, H), dtype=torch.float32, device=dev)
        wsb_bytes = lmh.lmhead_logprob_bwd_workspace_size(T, H, V)
        if a.bwd_workspace_mb:
            wsb_bytes = a.bwd_workspace_mb << 20
        wsb = torch.empty(wsb_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    extended = tau != 1.0 or wl.sum_p2 or wl.shards > 1 or wl.entropy_grad
    if wl.shards > 1:   # every shard's records, once, so the fold reads real data
        for s0, s1 in shards:
            lmh.lmhead_logprob_fwd_partials_ex(h, w[s0:s1], y, tau, s0, V, wl.sum_p2, ws, stream)

    if a.copy_bytes:
        src = torch.empty(a.copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    nev = 4 if wl.backward else 3

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        if extended:
            lmh.lmhead_logprob_fwd_partials_ex(h, w[v0:v1], y, tau, v0, V, wl.sum_p2, ws, stream)
        else:
            lmh.lmhead_logprob_fwd_partials(h, w, y, ws, stream)
        if evs is not None:
            evs[1].record(stream)
        if extended:
            lmh.lmhead_logprob_fwd_finalize_ex(y, T, H, V, lp, ent, lse, p2, ws, stream)
        else:
            lmh.lmhead_logprob_fwd_finalize(y, T, H, V, lp, ent, lse, ws, stream)
        if evs is not None:
            evs[2].record(stream)
        if wl.backward:
            if extended:
                lmh.lmhead_logprob_bwd_ex(h, w, y, tau, g, lse, ge, ent if ge is not None else None, gh, gw, False,
                                          wsb, stream)
            else:
                lmh.lmhead_logprob_bwd(h, w, y, g, lse, gh, gw, False, wsb, stream)
            if evs is not None:
                evs[3].record(stream)

    print(f"[bench] warmup {a.warmup}", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(a.steps)]
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [e[0].elapsed_time(e[-1]) for e in evs]               # ms, each step on the stream
    k1 = sum(e[0].elapsed_time(e[1]) for e in evs) / a.steps       # ms, stage 1 (logit tiles + records)
    k2 = sum(e[1].elapsed_time(e[2]) for e in evs) / a.steps       # ms, stage 2 (fold)
    kb = sum(e[2].elapsed_time(e[3]) for e in evs) / a.steps if wl.backward else 0.0
    ms = wall * 1e3 / a.steps
    fwd_flops = 2.0 * T * H * Vp                          # the partials stage's logit tiles
    flops = 2.0 * T * H * V * (4.0 if wl.backward else 1.0) if wl.shards == 1 else fwd_flops
    alg_bytes = 2.0 * Vp * H + 2.0 * T * H + 12.0 * T     # W (or its shard) once, h once, labels + outputs
    k1_tflops = fwd_flops / (k1 * 1e-3) / 1e12
    k1_gbs = alg_bytes / (k1 * 1e-3) / 1e9
    # W (2VH bytes) streamed once for 2TVH flops: T flop/B; below the ridge the kernel is HBM-bound
    hbm_bound = T < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(a.workload) if a.fwd_workspace == "fast" else None
    if T <= 128:
        kname = "fwd_partials_kernel"
    elif (a.fwd_workspace == "fast"
          and lmh.lmhead_logprob_fwd_workspace_size(T, H, Vp) > lmh.lmhead_logprob_fwd_workspace_size_min(T, H, Vp)):
        kname = "fwd_partials_sk_kernel"       # the K-split schedule (one token tile, few tiles per CU)
    else:
        kname = "fwd_partials_persistent_kernel"
    if hbm_bound:
        roof = {"bound": "hbm", "kernel": kname, "achieved": k1_gbs, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": k1_gbs / PEAK_HBM_GBS, "traffic": traffic}
    else:
        roof = {"bound": "mfma", "kernel": kname, "achieved": k1_tflops, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": k1_tflops / PEAK_BF16_TFLOPS, "traffic": traffic}
    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": float(np.median(step_ms)),
        "ms_per_step_mean_events": float(np.mean(step_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": a.workload, "T": T, "H": H, "V": V, "entropy": bool(wl.entropy),
                   "backward": bool(wl.backward),
                   **({"temperature": tau} if tau != 1.0 else {}), **({"sum_p2": True} if wl.sum_p2 else {}),
                   **({"entropy_grad": True} if wl.entropy_grad else {}),
                   **({"bwd_workspace_bytes": wsb_bytes} if wl.backward else {}),
                   **({"fwd_workspace": "min"} if a.fwd_workspace == "min" else {}),
                   **({"vocab_shard": [v0, v1], "shards": wl.shards} if wl.shards > 1 else {})},
        "tflops": flops / (ms * 1e-3) / 1e12,
        "pct_bf16_mfma_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stage_ms": {"fwd_partials": k1, "fwd_finalize": k2, **({"bwd": kb} if wl.backward else {})},
        "roofline": roof,
        "hbm_gbs_algorithmic": alg_bytes / (k1 * 1e-3) / 1e9,
        "kernel_sources_digest": kernel_sources_digest(),
    }
    if wl.backward:
        out["bwd_tflops"] = 6.0 * T * H * V / (kb * 1e-3) / 1e12
    if a.cpu_sample_rows != 0:
        print(f"[bench] timing the CPU oracle ({'automatic sample' if a.cpu_sample_rows < 0 else a.cpu_sample_rows} "
              "rows)", file=sys.stderr, flush=True)
        out["cpu_baseline"], ref = cpu_baseline(x, min(a.cpu_sample_rows, T), a.workload, tau, wl.sum_p2)
        # the timed run's own outputs (the last timed step's) against the oracle on the same rows
        out["parity"] = parity(ref, lp.cpu().double().numpy(), None if ent is None else ent.cpu().double().numpy())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
