"""Benchmark of the MoE layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one ``moe_forward`` call (router -> dispatch -> gate/up GEMM + SwiGLU -> down GEMM
-> combine) over one batch of seeded synthetic inputs already resident in HBM.  The default
workload is the prefill-shaped layer (4096 tokens, hidden 4096, 128 experts, top-8, expert FFN
1536, bf16, router bias N(0,1)).  Prints one JSON line.

Besides the step time it measures, with events on the launch stream, the average duration of
the dominant kernel (the gate/up grouped GEMM, launched alone through ``moe_grouped_gemm`` on
the same routing) and reports it against the MI355X roofline, and it times the CPU oracle on a
bounded sub-batch of the same workload as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E
METRIC = "MoE layer tokens/s at 1 GPU; % MFMA peak (prefill) / % HBM BW (decode)"


def describe(wl) -> str:
    return ("%s: %d tokens, hidden %d, %d experts, top-%d, expert ffn %d, %s weights / %s activations"
            % (wl.name, wl.tokens, wl.hidden, wl.experts, wl.top_k, wl.ffn, wl.wdt, wl.act))


def bytes_per_weight(wdt: str) -> float:
    return {"f32": 4.0, "bf16": 2.0, "nvfp4": 0.5 + 1.0 / 16}[wdt]


def layer_work(wl, active: int):
    """Algorithmic FLOPs and HBM bytes of one layer call (intermediates excluded)."""
    act = 4 if wl.act == "f32" else 2
    flops = 2.0 * wl.tokens * wl.hidden * wl.experts + 6.0 * wl.hidden * wl.ffn * wl.assignments
    nbytes = (active * 3.0 * wl.hidden * wl.ffn * bytes_per_weight(wl.wdt)
              + wl.experts * wl.hidden * act + 2.0 * wl.tokens * wl.hidden * act)
    return flops, nbytes


def gate_up_work(wl, active: int):
    """Algorithmic FLOPs and bytes of one gate/up grouped-GEMM launch: weights of the active
    experts once, each token row once, the hid output once."""
    act = 4 if wl.act == "f32" else 2
    flops = 4.0 * wl.hidden * wl.ffn * wl.assignments
    nbytes = (active * 2.0 * wl.ffn * wl.hidden * bytes_per_weight(wl.wdt)
              + wl.tokens * wl.hidden * act + wl.assignments * wl.ffn * act)
    return flops, nbytes


def cpu_baseline(wl, inputs, budget_s: float):
    """The oracle (as it stands) on a sub-batch of the same workload's tokens."""
    import numpy as np

    from oracle import oracle as O

    O.build()
    sub = dict(inputs)
    n = 8
    spent = 0.0
    while True:
        sub["x"] = inputs["x"][:n]
        t0 = time.perf_counter()
        O.forward(sub, wl.top_k, wl.wdt, wl.ffn, wl.renormalize)
        spent = time.perf_counter() - t0
        if spent >= budget_s / 4 or n >= wl.tokens:
            break
        n = min(wl.tokens, int(n * max(2.0, budget_s / 4 / max(spent, 1e-3))))
    return dict(value=n / spent, unit="tokens/s", cores=O.max_threads(), kind="oracle",
                sample="first %d of the %d tokens, whole layer (route, dispatch, expert FFNs, "
                       "combine) in fp64, %.1f s" % (n, wl.tokens, spent), seconds=spent)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this layer is built and measured on a single "
              "MI355X (no sharding, no collectives); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mixture_experts_layer_softmax_amd import lib, synth
    from mixture_experts_layer_softmax_amd.layer import MoELayer

    wl = synth.WORKLOADS[args.workload]
    print("[bench] generating %s" % describe(wl), file=sys.stderr, flush=True)
    inputs = synth.generate(wl)
    torch.cuda.set_device(0)
    layer = MoELayer.from_workload(wl, inputs, device="cuda:0")
    x = layer.act_tensor(inputs["x"])
    y = layer.empty_act(wl.tokens, wl.hidden)

    # routing of this batch (also gives the realised number of active experts)
    _, dbg = layer.forward(x, debug=True)
    torch.cuda.synchronize()
    counts = dbg["counts"].cpu().numpy()
    active = int((counts > 0).sum())

    print("[bench] warmup %d, timed %d steps" % (args.warmup, args.steps), file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer.forward(x, y=y)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        layer.forward(x, y=y)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # the dominant kernel alone: gate/up grouped GEMM on the same routing, same stream
    p = layer.problem_for(wl.tokens)
    ws = layer.workspace(wl.tokens)
    hid = layer.empty_act(wl.assignments, wl.ffn)
    for _ in range(2):
        lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x, dbg["sorted_token"], dbg["offsets"],
                         layer.weights, hid, ws)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x, dbg["sorted_token"], dbg["offsets"],
                         layer.weights, hid, ws)
    g1.record()
    torch.cuda.synchronize()
    gemm1_ms = g0.elapsed_time(g1) / args.steps  # includes the tiny tile-list kernel

    flops, nbytes = layer_work(wl, active)
    gflops, gbytes = gate_up_work(wl, active)
    t_mfma, t_hbm = gflops / PEAK_BF16_FLOPS, gbytes / PEAK_HBM_BYTES
    if t_hbm >= t_mfma:
        roof = dict(bound="hbm", achieved=gbytes / (gemm1_ms * 1e-3) / 1e9, peak=PEAK_HBM_BYTES / 1e9,
                    unit="GB/s")
    else:
        roof = dict(bound="mfma", achieved=gflops / (gemm1_ms * 1e-3) / 1e12,
                    peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "gemm_bf16_kernel gate/up + SwiGLU (%s weights)" % wl.wdt
    roof["kernel_ms"] = gemm1_ms

    tok_s = wl.tokens / (ms_per_step * 1e-3)
    out = dict(metric=METRIC, value=tok_s, unit="tokens/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype=wl.act, data="synthetic (seeded)",
               config=dict(workload=describe(wl), tokens=wl.tokens, hidden=wl.hidden,
                           experts=wl.experts, top_k=wl.top_k, ffn=wl.ffn, weights=wl.wdt,
                           active_experts=active, max_expert_rows=int(counts.max())),
               layer_tflops=flops / (ms_per_step * 1e-3) / 1e12,
               layer_mfma_frac=flops / (ms_per_step * 1e-3) / PEAK_BF16_FLOPS,
               layer_hbm_frac=nbytes / (ms_per_step * 1e-3) / PEAK_HBM_BYTES,
               wall_s=wall, roofline=roof)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, inputs, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
