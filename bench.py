"""Benchmark of the MoE layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one ``moe_forward`` call (router -> dispatch -> gate/up GEMM + SwiGLU -> down GEMM
-> combine) over one batch of seeded synthetic inputs already resident in HBM.  The default
workload is the prefill-shaped layer (4096 tokens, hidden 4096, 128 experts, top-8, expert FFN
1536, bf16, router bias N(0,1)); ``--workload`` selects another one (tiny, decode1, decode8,
decode64, nvfp4_decode, nvfp4_prefill).  Prints one JSON line.

Timing: W untimed steps, then K steps between two events on the launch stream.  Workloads
whose selected weights are small enough to stay cached between steps (under 1.5 GiB) read a
1 GiB buffer before every timed step and time each step with its own event pair, so that
weights come from HBM; the flush is outside the timed intervals (``--flush-mode write``
overwrites the buffer instead, for comparison).

Besides the step time it measures, with events on the same stream, the average duration of
the dominant kernel (the gate/up grouped GEMM, launched alone through ``moe_grouped_gemm`` on
the same routing) and reports it against the MI355X roofline.  ``traffic`` (HBM bytes per
launch of that kernel) comes from the counter summary under profiles/ when it was taken on the
current kernel source, else null.  The CPU oracle is timed on a bounded sub-batch of the same
workload as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E
METRIC = "MoE layer tokens/s at 1 GPU; % MFMA peak (prefill) / % HBM BW (decode)"
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_softmax_amd", "csrc", "gemm.hip")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def describe(wl) -> str:
    return ("%s: %d tokens, hidden %d, %d experts, top-%d, expert ffn %d, %s weights / %s activations"
            % (wl.name, wl.tokens, wl.hidden, wl.experts, wl.top_k, wl.ffn, wl.wdt, wl.act))


def bytes_per_weight(wdt: str) -> float:
    return {"f32": 4.0, "bf16": 2.0, "nvfp4": 0.5 + 1.0 / 16}[wdt]


def layer_work(wl, active: int):
    """Algorithmic FLOPs and HBM bytes of one layer call: router + expert FFN FLOPs; the
    active experts' weights once, the router weight, tokens in and out (intermediates
    excluded: the method need not send them to HBM)."""
    act = 4 if wl.act == "f32" else 2
    flops = 2.0 * wl.tokens * wl.hidden * wl.experts + 6.0 * wl.hidden * wl.ffn * wl.assignments
    nbytes = (active * 3.0 * wl.hidden * wl.ffn * bytes_per_weight(wl.wdt)
              + wl.experts * wl.hidden * act + 2.0 * wl.tokens * wl.hidden * act)
    return flops, nbytes


def gate_up_work(wl, active: int):
    """Algorithmic FLOPs and bytes of one gate/up grouped-GEMM launch: the active experts'
    gate/up weights once, each token row once, the hid output once."""
    act = 4 if wl.act == "f32" else 2
    flops = 4.0 * wl.hidden * wl.ffn * wl.assignments
    nbytes = (active * 2.0 * wl.ffn * wl.hidden * bytes_per_weight(wl.wdt)
              + wl.tokens * wl.hidden * act + wl.assignments * wl.ffn * act)
    return flops, nbytes


def source_hash() -> str:
    return hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per gate/up launch from the committed counter summary, if it is current."""
    try:
        d = json.load(open(TRAFFIC))
    except (OSError, ValueError):
        return None
    e = d.get(workload)
    if not e or e.get("gemm_source_sha256_16") != source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(wl, inputs, budget_s: float):
    """The oracle (as it stands) on a sub-batch of the same workload's tokens."""
    from oracle import oracle as O

    O.build()
    sub = dict(inputs)
    n = min(8, wl.tokens)
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


def measured_peaks(torch, lib):
    """What this machine sustains: the bf16 MFMA probe (8 blocks per CU) and a 4 GiB HBM read
    stream (moe_probe.h), best of three timed runs each, on the current stream."""
    def best(fn, runs=3):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(runs):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            work = fn()
            b.record()
            torch.cuda.synchronize()
            t.append((work, a.elapsed_time(b) * 1e-3))
        return max(w / s for w, s in t)

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(8 * cus, dtype=torch.float32, device="cuda:0")
    flops = best(lambda: lib.probe_mfma_bf16(8 * cus, 20000, sink))
    buf = torch.empty(4 * 2 ** 30, dtype=torch.uint8, device="cuda:0")
    word = torch.empty(1, dtype=torch.int32, device="cuda:0")
    rate = best(lambda: lib.probe_read(buf, word))
    del buf
    return dict(mfma_bf16_tflops=flops / 1e12, hbm_read_gbs=rate / 1e9,
                probes="bf16 MFMA loop, %d blocks x 4 wavefronts x 20000 x 8 v_mfma_f32_16x16x32_bf16; "
                       "read stream over 4 GiB" % (8 * cus))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--flush", choices=("auto", "on", "off"), default="auto")
    ap.add_argument("--flush-mode", choices=("read", "write"), default="read",
                    help="evict caches by reading (default) or by writing a 1 GiB buffer")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured-peak probes (bf16 MFMA loop, 4 GiB read stream)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one 512 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this layer is built and measured on a single "
              "MI355X (no sharding, no collectives); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        return 2

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
    w_bytes = active * 3.0 * wl.hidden * wl.ffn * bytes_per_weight(wl.wdt)
    flush = args.flush == "on" or (args.flush == "auto" and w_bytes < 1.5 * 2 ** 30)
    scratch = torch.ones(2 ** 30, dtype=torch.uint8, device="cuda:0") if flush else None
    scratch_word = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def evict():
        # Reading 1 GiB of other data displaces the layer's weights from L2 and the 256 MiB
        # Infinity Cache.  Writing it instead would leave dirty lines whose write-back lands
        # inside the next timed interval and competes with the weight stream.
        if args.flush_mode == "read":
            lib.probe_read(scratch, scratch_word)
        else:
            scratch.fill_(1)

    def timed(fn, steps):
        """Mean ms per call of fn over `steps` calls on the current stream."""
        if not flush:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            evict()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / steps

    print("[bench] warmup %d, timed %d steps%s" % (args.warmup, args.steps, " (flushed)" if flush else ""),
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer.forward(x, y=y)
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_per_step = timed(lambda: layer.forward(x, y=y), args.steps)
    wall = time.perf_counter() - t0

    # the dominant kernel alone: gate/up grouped GEMM on the same routing, same stream
    p = layer.problem_for(wl.tokens)
    ws = layer.workspace(wl.tokens)
    hid = layer.empty_act(wl.assignments, wl.ffn)
    gemm1 = lambda: lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x, dbg["sorted_token"], dbg["offsets"],
                                     layer.weights, hid, ws)
    for _ in range(2):
        gemm1()
    torch.cuda.synchronize()
    gemm1_ms = timed(gemm1, args.steps)  # includes the ~5 us tile-list kernel it launches first

    peaks = None if args.no_probes else measured_peaks(torch, lib)

    if args.calibration_copy:
        a = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

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
    if peaks:
        mp = peaks["hbm_read_gbs"] if roof["bound"] == "hbm" else peaks["mfma_bf16_tflops"]
        roof["frac_measured"] = roof["achieved"] / mp
    roof["traffic"] = measured_traffic(wl.name)
    roof["kernel"] = "grouped gate/up GEMM + SwiGLU (%s weights)" % wl.wdt
    roof["kernel_ms"] = gemm1_ms
    roof["algorithmic_bytes"] = gbytes
    roof["algorithmic_flops"] = gflops

    tok_s = wl.tokens / (ms_per_step * 1e-3)
    out = dict(metric=METRIC, value=tok_s, unit="tokens/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype=wl.act, data="synthetic (seeded)",
               config=dict(workload=describe(wl), tokens=wl.tokens, hidden=wl.hidden,
                           experts=wl.experts, top_k=wl.top_k, ffn=wl.ffn, weights=wl.wdt,
                           active_experts=active, max_expert_rows=int(counts.max()),
                           cache_flushed=bool(flush),
                           flush_mode=args.flush_mode if flush else None),
               layer_tflops=flops / (ms_per_step * 1e-3) / 1e12,
               layer_mfma_frac=flops / (ms_per_step * 1e-3) / PEAK_BF16_FLOPS,
               layer_hbm_frac=nbytes / (ms_per_step * 1e-3) / PEAK_HBM_BYTES,
               wall_s=wall, roofline=roof)
    if peaks:
        out["measured_peaks"] = peaks
        out["layer_mfma_frac_measured"] = flops / (ms_per_step * 1e-3) / (peaks["mfma_bf16_tflops"] * 1e12)
        out["layer_hbm_frac_measured"] = nbytes / (ms_per_step * 1e-3) / (peaks["hbm_read_gbs"] * 1e9)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, inputs, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
