"""Benchmark of the MoE layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload nvfp4_prefill]

A step is one ``moe_forward`` call (router -> dispatch -> gate/up GEMM + SwiGLU -> down GEMM
-> combine) over one batch of seeded synthetic inputs already resident in HBM.  The default
workload is the largest single-GPU layer: 8192 tokens, hidden 4096, 256 experts, top-8, expert
FFN 2048, 4-bit E2M1 weights with one E4M3 scale per 16 (decoded exactly to bf16 for the bf16
matrix cores), bf16 activations, router bias on a 10 % hot set that receives half of the
assignments.  ``--workload`` selects another one (tiny, prefill, decode1, decode8, decode64,
nvfp4_decode, prefill6000, mxfp8_prefill, mxfp4_prefill, mxfp8_decode64, mxfp4_decode64).
Prints one JSON line.

Shapes of "Hosting Qwen on Blackwell" (sections Prefill, Expert Parallel and the grouped MoE
GEMM benchmark there):
  --workload prefill6000 [--ep-size N --ep-rank r]
        the ~6000-token prefill (about 375 rows per expert); with N > 1, the share of rank r
        of N expert-parallel ranks: every token is routed, the rank holds experts
        [r E/N, (r+1) E/N) and returns its partial output (the all-reduce that sums the
        partial outputs is the caller's and is not timed).  Any workload takes --ep-size.
  --workload grouped1 [--ep-size N]
        the grouped MoE GEMM with every expert given one token: gate/up + SwiGLU then down
        through moe_grouped_gemm on E/N experts (hidden 4096, expert ffn 1536, bf16), one row
        each; reports the latency of the pair.

Timing: W untimed steps, then K steps bracketed by a device synchronisation on both sides,
with an event recorded on the launch stream before and after every step, so that the line
carries the mean (``ms_per_step``, whole bracket / K) and the per-step median, p10 and p90.
Workloads whose selected weights are small enough to stay cached between steps (under 1.5 GiB)
read a 1 GiB buffer before every timed step, outside the step's event pair, so that weights
come from HBM (``--flush-mode write`` overwrites the buffer instead, for comparison).

Besides the step time it measures, with an event pair per launch on the same stream, the
duration of the dominant kernel (the gate/up grouped GEMM, launched alone through
``moe_grouped_gemm`` on the same routing, K times) and reports it against the MI355X roofline.  ``traffic`` (HBM bytes per
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
PEAK_FP8_FLOPS = 5.0e15    # MI355X dense fp8 MFMA (the MXFP8 layer's block-scaled products)
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E
METRIC = "MoE layer tokens/s at 1 GPU; % MFMA peak (prefill) / % HBM BW (decode)"
CSRC = os.path.join(ROOT, "mixture_experts_layer_softmax_amd", "csrc")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def describe(wl) -> str:
    return ("%s: %d tokens, hidden %d, %d experts, top-%d, expert ffn %d, %s weights / %s activations"
            % (wl.name, wl.tokens, wl.hidden, wl.experts, wl.top_k, wl.ffn, wl.wdt, wl.act))


def bytes_per_weight(wdt: str) -> float:
    return {"f32": 4.0, "bf16": 2.0, "nvfp4": 0.5 + 1.0 / 16, "mxfp8": 1.0 + 1.0 / 32,
            "mxfp4": 0.5 + 1.0 / 32}[wdt]


def mfma_peak(wl) -> float:
    """Dense MFMA peak of the dtype the expert GEMMs multiply in (NVFP4 is decoded to bf16;
    MXFP4 weights multiply fp8 activations, priced at the fp8 rate)."""
    return PEAK_FP8_FLOPS if wl.wdt.startswith("mx") else PEAK_BF16_FLOPS


def layer_work(wl, active: int, rows: int):
    """Algorithmic FLOPs and HBM bytes of one layer call: router + expert FFN FLOPs of the
    `rows` dispatched assignments; the active experts' weights once, the router weight,
    tokens in and out (intermediates excluded: the method need not send them to HBM)."""
    act = 4 if wl.act == "f32" else 2
    flops = 2.0 * wl.tokens * wl.hidden * wl.experts + 6.0 * wl.hidden * wl.ffn * rows
    nbytes = (active * 3.0 * wl.hidden * wl.ffn * bytes_per_weight(wl.wdt)
              + wl.experts * wl.hidden * act + 2.0 * wl.tokens * wl.hidden * act)
    return flops, nbytes


def gate_up_work(wl, active: int, rows: int, tokens_read: int):
    """Algorithmic FLOPs and bytes of one gate/up grouped-GEMM launch over `rows` dispatched
    rows: the active experts' gate/up weights once and each token row it reads once.  The hid
    it writes is an intermediate of the layer and is not counted, as in layer_work."""
    act = 4 if wl.act == "f32" else 2
    flops = 4.0 * wl.hidden * wl.ffn * rows
    nbytes = (active * 2.0 * wl.ffn * wl.hidden * bytes_per_weight(wl.wdt)
              + tokens_read * wl.hidden * act)
    return flops, nbytes


def kernel_source(wdt: str) -> list:
    """Source files of the gate/up GEMM kernel of a weight format (the kernel file and the
    headers its kernels are built from)."""
    kern = ["mx.hip"] if wdt.startswith("mx") else ["gemm.hip", "gemv.h"]
    return [os.path.join(CSRC, f) for f in kern + ["lds_dma.h", "device.h", "launch.h"]]


def source_hash(paths) -> str:
    """First 16 hex digits of the sha256 of the files' contents, concatenated in order."""
    h = hashlib.sha256()
    for p in ([paths] if isinstance(paths, str) else paths):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, wdt: str):
    """HBM bytes per gate/up launch from the committed counter summary, if it was taken on the
    current source of that kernel."""
    try:
        d = json.load(open(TRAFFIC))
    except (OSError, ValueError):
        return None
    e = d.get(workload)
    if not e or e.get("gemm_source_sha256_16") != source_hash(kernel_source(wdt)):
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(wl, inputs, budget_s: float, held=None):
    """The oracle (as it stands) on a sub-batch of the same workload's tokens."""
    from oracle import oracle as O

    O.build()
    sub = dict(inputs)
    n = min(8, wl.tokens)
    while True:
        sub["x"] = inputs["x"][:n]
        t0 = time.perf_counter()
        O.forward(sub, wl.top_k, wl.wdt, wl.ffn, wl.renormalize, held=held)
        spent = time.perf_counter() - t0
        if spent >= budget_s / 2 or n >= wl.tokens:  # a final sample of 10-20 s at the default
            break
        n = min(wl.tokens, int(n * max(2.0, budget_s / 2 / max(spent, 1e-3))))
    out = dict(value=n / spent, unit="tokens/s", cores=O.max_threads(), kind="oracle",
               sample="first %d of the %d tokens, whole layer (route, dispatch, expert FFNs, "
                      "combine) in fp64, %.1f s" % (n, wl.tokens, spent), seconds=spent)
    if wl.tokens <= 64:  # decode-sized batches: also one thread, median of three runs
        threads = O.max_threads()
        O.set_threads(1)
        try:
            runs = []
            for _ in range(3):
                t0 = time.perf_counter()
                O.forward(sub, wl.top_k, wl.wdt, wl.ffn, wl.renormalize, held=held)
                runs.append(time.perf_counter() - t0)
        finally:
            O.set_threads(threads)
        one = sorted(runs)[1]
        out["single_thread"] = dict(value=n / one, unit="tokens/s", cores=1, seconds=one,
                                    sample="the same %d tokens, median of 3 runs" % n)
    return out


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
    rate = best(lambda: lib.probe_read(buf, word, nontemporal=True))
    del buf
    return dict(mfma_bf16_tflops=flops / 1e12, hbm_read_gbs=rate / 1e9,
                probes="bf16 MFMA loop, %d blocks x 4 wavefronts x 20000 x 8 v_mfma_f32_16x16x32_bf16; "
                       "non-temporal read stream over 4 GiB" % (8 * cus))


def percentile(v, q):
    """Linear-interpolated percentile q (0..100) of the list v."""
    v = sorted(v)
    if not v:
        return None
    x = (len(v) - 1) * q / 100.0
    i = int(x)
    j = min(i + 1, len(v) - 1)
    return v[i] + (v[j] - v[i]) * (x - i)


def step_stats(per_step):
    """Mean, median, p10 and p90 (ms) of a list of per-call durations (ms)."""
    return dict(mean=sum(per_step) / len(per_step), median=percentile(per_step, 50),
                p10=percentile(per_step, 10), p90=percentile(per_step, 90), n=len(per_step))


def make_timer(torch, lib, flush: bool, flush_mode: str):
    """timed(fn, steps) -> dict(mean, median, p10, p90, n) in ms per call of fn on the current
    stream, from an event recorded before and after every call.  Without `flush` the calls run
    back to back (event i+1 both ends call i and starts call i+1, so the mean is the whole
    bracket over the calls); with `flush` caches are evicted before every call, outside its
    event pair."""
    scratch = torch.ones(2 ** 30, dtype=torch.uint8, device="cuda:0") if flush else None
    scratch_word = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def evict():
        # Reading 1 GiB of other data displaces the layer's weights from L2 and the 256 MiB
        # Infinity Cache.  Writing it instead would leave dirty lines whose write-back lands
        # inside the next timed interval and competes with the weight stream.
        if flush_mode == "read":
            lib.probe_read(scratch, scratch_word)
        else:
            scratch.fill_(1)

    def timed(fn, steps):
        if not flush:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            evs[0].record()
            for i in range(steps):
                fn()
                evs[i + 1].record()
            torch.cuda.synchronize()
            per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
            out = step_stats(per)
            out["mean"] = evs[0].elapsed_time(evs[steps]) / steps
            return out
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            evict()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return step_stats([a.elapsed_time(b) for a, b in evs])

    timed.scratch, timed.scratch_word = scratch, scratch_word
    return timed


def _find_clocks(d):
    """The gfx / memory clock entries (current, min, max; MHz) anywhere in amd-smi's JSON."""
    if isinstance(d, list):
        for v in d:
            c = _find_clocks(v)
            if c:
                return c
        return None
    if not isinstance(d, dict):
        return None
    if "gfx_0" in d or "mem_0" in d:
        out = {}
        for key in ("gfx_0", "mem_0", "fclk_0", "socclk_0"):
            v = d.get(key)
            if isinstance(v, dict):
                out[key] = {f: (v[f].get("value") if isinstance(v[f], dict) else v[f])
                            for f in ("clk", "min_clk", "max_clk") if f in v}
        return out
    for v in d.values():
        c = _find_clocks(v)
        if c:
            return c
    return None


def platform_info(torch, skip_clocks=False):
    """ROCm / HIP versions, the device name, and the GPU clocks as amd-smi reports them before
    the run (a child process; None where the tool is missing, says nothing parseable, runs under
    a profiler, or skip_clocks is set).  The current clock is sampled at idle; max_clk is the
    clock cap the timed work runs under."""
    import subprocess

    info = dict(hip=getattr(torch.version, "hip", None), torch=torch.__version__)
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    try:
        info["device"] = torch.cuda.get_device_name(0)
    except Exception:  # pragma: no cover
        info["device"] = None
    clocks = None
    if skip_clocks or any(k.startswith("ROCPROF") for k in os.environ):
        # under a profiler the child would load the profiler's tool, which opens the GPU in the
        # amd-smi launcher before it starts its interpreter: leave the clocks out there
        info["clocks_mhz_before_run"] = None
        return info
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True,
                           text=True, timeout=30)
        if r.returncode == 0 and r.stdout.strip():
            clocks = _find_clocks(json.loads(r.stdout))
    except (OSError, ValueError, subprocess.SubprocessError):
        clocks = None
    info["clocks_mhz_before_run"] = clocks  # sampled while the GPU idles: max_clk is the cap
    return info


def bench_grouped1(args) -> int:
    """Grouped MoE GEMM with every expert given one token ("Hosting Qwen on Blackwell": the
    grouped GEMM benchmark across expert-parallel configurations activates every expert with a
    single token).  One rank of --ep-size holds E/N experts with one row each; a step is the
    gate/up + SwiGLU launch and the down launch of moe_grouped_gemm."""
    import numpy as np
    import torch

    from mixture_experts_layer_softmax_amd import lib, synth
    from mixture_experts_layer_softmax_amd.layer import MoELayer

    E, H, F = 128, 4096, 1536
    if E % args.ep_size:
        print("--ep-size must divide the %d experts" % E, file=sys.stderr)
        return 2
    n = E // args.ep_size
    b = args.ep_rank * n
    wl = synth.Workload("grouped1", n, H, E, 1, F, "bf16", "bf16", 707, "none")
    print("[bench] grouped GEMM, one token for each of experts [%d, %d) of %d" % (b, b + n, E),
          file=sys.stderr, flush=True)
    inputs = synth.generate(wl, experts=range(b, b + n))
    torch.cuda.set_device(0)
    held = dict(expert_begin=b, local_experts=n) if n < E else {}
    layer = MoELayer.from_workload(wl, inputs, device="cuda:0", **held)
    p = layer.problem_for(n)
    ws = layer.workspace(n)
    x = layer.act_tensor(inputs["x"])  # row i is the token of expert b + i
    offsets = torch.from_numpy(np.clip(np.arange(E + 1) - b, 0, n).astype(np.int32)).cuda()
    hid = layer.empty_act(n, F)
    yp = layer.empty_act(n, H)

    def step():
        lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x, None, offsets, layer.weights, hid, ws)
        lib.grouped_gemm(p, lib.DOWN, hid, None, offsets, layer.weights, yp, ws)

    w_bytes = n * 3.0 * H * F * 2
    flush = args.flush == "on" or (args.flush == "auto" and w_bytes < 1.5 * 2 ** 30)
    timed = make_timer(torch, lib, flush, args.flush_mode)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st = timed(step, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = st["mean"]
    nbytes = w_bytes + n * (H + F + F + H) * 2.0  # weights once; x, hid out/in, y_perm out
    flops = n * 6.0 * H * F
    gbs = nbytes / (ms * 1e-3) / 1e9
    peaks = None if args.no_probes else measured_peaks(torch, lib)
    roof = dict(bound="hbm", achieved=gbs, peak=PEAK_HBM_BYTES / 1e9, unit="GB/s",
                frac=gbs * 1e9 / PEAK_HBM_BYTES, traffic=None,
                kernel="grouped gate/up + down GEMM pair, one row per expert", kernel_ms=ms,
                algorithmic_bytes=nbytes, algorithmic_flops=flops)
    if peaks:
        roof["frac_measured"] = gbs / peaks["hbm_read_gbs"]
    out = dict(metric="grouped MoE GEMM latency, every expert given one token", value=ms * 1e3,
               unit="us", n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=ms,
               step_ms=dict(median=st["median"], p10=st["p10"], p90=st["p90"]),
               higher_is_better=False, scaling="weak", vs_baseline=None, dtype="bf16",
               data="synthetic (seeded)",
               config=dict(workload="grouped1: one token for each of %d experts (rank %d of %d "
                                    "expert-parallel ranks over %d experts), hidden %d, expert "
                                    "ffn %d, bf16" % (n, args.ep_rank, args.ep_size, E, H, F),
                           experts=n, hidden=H, ffn=F, ep_size=args.ep_size, ep_rank=args.ep_rank,
                           cache_flushed=bool(flush)),
               wall_s=wall, roofline=roof)
    if peaks:
        out["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        from oracle import oracle as O

        O.build()
        t1 = time.perf_counter()
        O.expert_rows(inputs, "bf16", F, np.arange(n), np.arange(n))
        spent = time.perf_counter() - t1
        out["cpu_baseline"] = dict(value=spent * 1e6, unit="us", cores=O.max_threads(), kind="oracle",
                                   sample="all %d rows: gate/up, SwiGLU and down in fp64" % n,
                                   seconds=spent)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="nvfp4_prefill")
    ap.add_argument("--flush", choices=("auto", "on", "off"), default="auto")
    ap.add_argument("--flush-mode", choices=("read", "write"), default="read",
                    help="evict caches by reading (default) or by writing a 1 GiB buffer")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured-peak probes (bf16 MFMA loop, 4 GiB read stream)")
    ap.add_argument("--no-clocks", action="store_true",
                    help="do not start amd-smi for the GPU clocks (also skipped under rocprofv3)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one 512 MiB device copy (counter calibration)")
    ap.add_argument("--ep-size", type=int, default=1,
                    help="expert-parallel degree whose one-rank share is measured (one GPU)")
    ap.add_argument("--ep-rank", type=int, default=0)
    ap.add_argument("--path", choices=("auto", "prefill", "decode", "fused"), default="auto",
                    help="kernel family of moe_forward (fused: the single-launch decode kernel)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this layer is built and measured on a single "
              "MI355X (no collectives); --gpus %d is not supported.  One expert-parallel rank's "
              "share is measured with --ep-size N --ep-rank r." % args.gpus, file=sys.stderr)
        return 2
    if args.ep_size < 1 or not 0 <= args.ep_rank < args.ep_size:
        print("--ep-rank must lie in [0, --ep-size)", file=sys.stderr)
        return 2
    if args.workload == "grouped1":
        return bench_grouped1(args)

    import torch

    from mixture_experts_layer_softmax_amd import lib, synth
    from mixture_experts_layer_softmax_amd.layer import MoELayer

    if args.workload not in synth.WORKLOADS:
        print("unknown workload %r (one of: %s, grouped1)" % (args.workload, ", ".join(synth.WORKLOADS)),
              file=sys.stderr)
        return 2
    wl = synth.WORKLOADS[args.workload]
    plat = platform_info(torch, args.no_clocks)
    held = None
    if args.ep_size > 1:
        if wl.experts % args.ep_size:
            print("--ep-size must divide the %d experts" % wl.experts, file=sys.stderr)
            return 2
        n = wl.experts // args.ep_size
        held = (args.ep_rank * n, n)
    print("[bench] generating %s%s" % (describe(wl), "" if held is None else
          ", experts [%d, %d) of rank %d/%d" % (held[0], held[0] + held[1], args.ep_rank, args.ep_size)),
          file=sys.stderr, flush=True)
    inputs = synth.generate(wl, experts=None if held is None else range(held[0], held[0] + held[1]))
    torch.cuda.set_device(0)
    layer = MoELayer.from_workload(wl, inputs, device="cuda:0", path=args.path,
                                   expert_begin=0 if held is None else held[0],
                                   local_experts=0 if held is None else held[1])
    x = layer.act_tensor(inputs["x"])
    y = layer.empty_act(wl.tokens, wl.hidden)

    # routing of this batch (also gives the realised number of active experts)
    _, dbg = layer.forward(x, debug=True)
    torch.cuda.synchronize()
    counts = dbg["counts"].cpu().numpy()
    active = int((counts > 0).sum())
    rows = int(counts.sum())  # dispatched rows: every assignment, or those of the held experts
    tokens_read = int(((dbg["inv_perm"].reshape(wl.tokens, wl.top_k) >= 0).any(1)).sum().item())
    w_bytes = active * 3.0 * wl.hidden * wl.ffn * bytes_per_weight(wl.wdt)
    flush = args.flush == "on" or (args.flush == "auto" and w_bytes < 1.5 * 2 ** 30)
    timed = make_timer(torch, lib, flush, args.flush_mode)

    print("[bench] warmup %d, timed %d steps%s" % (args.warmup, args.steps, " (flushed)" if flush else ""),
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer.forward(x, y=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps = timed(lambda: layer.forward(x, y=y), args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = steps["mean"]

    # the dominant kernel alone: the gate/up grouped GEMM on the same routing and stream, one
    # event pair per launch around the GEMM kernel (its tile list is built once, outside the
    # brackets; a read flush, when the workload takes one, runs before each launch outside its
    # bracket: moe_probe_grouped_gemm_times)
    p = layer.problem_for(wl.tokens)
    ws = layer.workspace(wl.tokens)
    hid = layer.empty_act(wl.assignments, wl.ffn)
    gemm1 = lambda: lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x, dbg["sorted_token"], dbg["offsets"],
                                     layer.weights, hid, ws)
    for _ in range(2):
        gemm1()
    torch.cuda.synchronize()
    print("[bench] dominant kernel, %d launches" % args.steps, file=sys.stderr, flush=True)
    if flush and args.flush_mode != "read":  # the old write flush: whole moe_grouped_gemm calls
        g1 = timed(gemm1, args.steps)
    else:
        per = lib.probe_grouped_gemm_times(p, lib.GATE_UP_SWIGLU, x, dbg["sorted_token"],
                                           dbg["offsets"], layer.weights, hid, ws, args.steps,
                                           flush=timed.scratch, flush_out=timed.scratch_word)
        g1 = step_stats(per)
    gemm1_ms = g1["mean"]

    peaks = None if args.no_probes else measured_peaks(torch, lib)

    if args.calibration_copy:
        a = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    flops, nbytes = layer_work(wl, active, rows)
    gflops, gbytes = gate_up_work(wl, active, rows, tokens_read)
    peak_mfma = mfma_peak(wl)
    t_mfma, t_hbm = gflops / peak_mfma, gbytes / PEAK_HBM_BYTES
    if t_hbm >= t_mfma:
        roof = dict(bound="hbm", achieved=gbytes / (gemm1_ms * 1e-3) / 1e9, peak=PEAK_HBM_BYTES / 1e9,
                    unit="GB/s")
    else:
        roof = dict(bound="mfma", achieved=gflops / (gemm1_ms * 1e-3) / 1e12,
                    peak=peak_mfma / 1e12, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    if peaks:
        if roof["bound"] == "hbm":
            roof["frac_measured"] = roof["achieved"] / peaks["hbm_read_gbs"]
        elif not wl.wdt.startswith("mx"):  # the probe measures the bf16 rate only
            roof["frac_measured"] = roof["achieved"] / peaks["mfma_bf16_tflops"]
    roof["traffic"] = measured_traffic(wl.name, wl.wdt) if held is None else None
    roof["kernel"] = "grouped gate/up GEMM + SwiGLU (%s weights%s)" % (
        wl.wdt, ", input quantization included" if wl.wdt.startswith("mx") else "")
    roof["kernel_ms"] = gemm1_ms
    roof["kernel_ms_median"] = g1["median"]
    roof["algorithmic_bytes"] = gbytes
    roof["algorithmic_flops"] = gflops

    tok_s = wl.tokens / (ms_per_step * 1e-3)
    out = dict(metric=METRIC, value=tok_s, unit="tokens/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=ms_per_step,
               step_ms=dict(median=steps["median"], p10=steps["p10"], p90=steps["p90"]),
               tokens_per_s_median=wl.tokens / (steps["median"] * 1e-3), higher_is_better=True,
               scaling="weak", vs_baseline=None,
               dtype={"mxfp8": "fp8", "mxfp4": "fp8 x fp4"}.get(wl.wdt, wl.act),
               data="synthetic (seeded)",
               config=dict(workload=describe(wl), tokens=wl.tokens, hidden=wl.hidden,
                           experts=wl.experts, top_k=wl.top_k, ffn=wl.ffn, weights=wl.wdt,
                           active_experts=active, max_expert_rows=int(counts.max()),
                           cache_flushed=bool(flush),
                           flush_mode=args.flush_mode if flush else None, path=args.path),
               layer_tflops=flops / (ms_per_step * 1e-3) / 1e12,
               layer_mfma_frac=flops / (ms_per_step * 1e-3) / peak_mfma,
               layer_hbm_frac=nbytes / (ms_per_step * 1e-3) / PEAK_HBM_BYTES,
               wall_s=wall, roofline=roof, platform=plat)
    if peaks:
        out["measured_peaks"] = peaks
        if not wl.wdt.startswith("mx"):
            out["layer_mfma_frac_measured"] = flops / (ms_per_step * 1e-3) / (peaks["mfma_bf16_tflops"] * 1e12)
        out["layer_hbm_frac_measured"] = nbytes / (ms_per_step * 1e-3) / (peaks["hbm_read_gbs"] * 1e9)
    if held is not None:
        out["config"].update(ep_size=args.ep_size, ep_rank=args.ep_rank,
                             held_experts=[held[0], held[0] + held[1]], dispatched_rows=rows,
                             output="partial (this rank's experts); the all-reduce is not timed")
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, inputs, args.cpu_budget, held)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
