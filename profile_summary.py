"""Summaries of rocprofv3 output for profiles/ (measurement tooling beside bench.py).

    python profile_summary.py kernels RUN_DIR TAG --last K --cmd "rocprofv3 ... -- python3 bench.py ..."
    python profile_summary.py traffic FETCH_DIR WRITE_DIR TAG WORKLOAD KERNEL SOURCE --cmd-fetch ... --cmd-write ...
    python profile_summary.py bench RUN_DIR
    python profile_summary.py counters TAG KERNEL DIR1 [DIR2 ...] --cmd ...

``kernels`` reads ``*_kernel_trace.csv`` of a ``rocprofv3 --kernel-trace`` run and writes
``profiles/TAG_kernel_stats.md``: per kernel, every launch (what ``--stats`` prints) and the last
K launches only.  bench.py launches each kernel of the forward K times in its timed steps after
its warm-up, and the gate/up GEMM K more times alone (the launches its roofline figure times),
so the last K launches of a kernel are the timed ones.

``bench`` reads the bench.py JSON lines saved as ``NAME.json`` beside ``NAME.cmd`` (the command
that printed it) in a directory, and writes ``profiles/bench_lines.md``: one row per run with
the headline figures, then every line in full.

``counters`` reads the ``*_counter_collection.csv`` of one or more ``rocprofv3 --pmc`` runs
(one counter pass each) and writes ``profiles/TAG_counters.md``: per counter, the average over
the kernel's launches of its value summed over the hardware instances, and the ratios that the
kernel analysis uses (MFMA busy share of the SIMD cycles, instructions per MFMA, LDS bank
conflicts per LDS instruction).

``traffic`` reads the ``*_counter_collection.csv`` of two ``rocprofv3 --pmc FETCH_SIZE`` /
``--pmc WRITE_SIZE`` runs of bench.py with ``--calibration-copy`` and writes
``profiles/TAG_traffic.md`` and the WORKLOAD entry of ``profiles/traffic.json``: the dominant
kernel's KiB per launch, scaled by what the same counter reads for the 512 MiB device copy at
the end of the run, with the hash of the kernel's source files (SOURCE: comma-separated paths
from the repository root, in the order bench.kernel_source lists them) so that bench.py stops
quoting it once the kernel changes.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit("no file matches %s" % pattern)
    return hits[0]


def _short(name: str, n: int = 110) -> str:
    return name if len(name) <= n else name[: n - 3] + "..."


def kernels(run_dir: str, tag: str, last: int, cmd: str) -> str:
    path = _one(os.path.join(run_dir, "**", "*kernel_trace.csv"))
    launches = collections.defaultdict(list)  # name -> [(start, duration us)]
    for r in csv.DictReader(open(path)):
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        launches[r["Kernel_Name"]].append((t0, (t1 - t0) / 1e3))
    total = sum(d for v in launches.values() for _, d in v)
    rows = []
    for name, v in launches.items():
        v.sort()
        d = [x for _, x in v]
        tail = d[-last:]
        rows.append((sum(d), name, d, tail))
    rows.sort(reverse=True)
    out = ["# Kernel trace: %s" % tag, "", "Command (run from the repository root on one MI355X):", "",
           "    " + cmd, "", "Then `python profile_summary.py kernels <run dir> %s --last %d`." % (tag, last), "",
           "Durations in microseconds.  *All*: every launch of the run (warm-up and untimed launches "
           "included, as `rocprofv3 --stats` counts them).  *Timed*: the last %d launches of each kernel: "
           "for the gate/up GEMM the launches of bench.py's kernel timing (its roofline figure), which "
           "follow the timed steps; for the other kernels the launches of the timed steps." % last, "",
           "| kernel | calls | all: average | timed: calls | timed: average | timed: median | timed: min | timed: max | share % |",
           "|---|---|---|---|---|---|---|---|---|"]
    for tot, name, d, tail in rows:
        out.append("| `%s` | %d | %.1f | %d | %.1f | %.1f | %.1f | %.1f | %.2f |" % (
            _short(name), len(d), sum(d) / len(d), len(tail), sum(tail) / len(tail),
            statistics.median(tail), min(tail), max(tail), 100.0 * tot / total))
    text = "\n".join(out) + "\n"
    os.makedirs(PROFILES, exist_ok=True)
    open(os.path.join(PROFILES, "%s_kernel_stats.md" % tag), "w").write(text)
    return text


def _per_launch(path: str):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def traffic(fetch_dir: str, write_dir: str, tag: str, workload: str, kernel: str, source: str,
            cmd_fetch: str, cmd_write: str) -> str:
    f = _per_launch(_one(os.path.join(fetch_dir, "**", "*counter_collection.csv")))
    w = _per_launch(_one(os.path.join(write_dir, "**", "*counter_collection.csv")))
    copy_f = max(f["__amd_rocclr_copyBuffer"])
    copy_w = max(w["__amd_rocclr_copyBuffer"])
    kf = [v for k, vs in f.items() if kernel in k for v in vs]
    kw = [v for k, vs in w.items() if kernel in k for v in vs]
    if not kf or not kw:
        raise SystemExit("kernel %r not found in the counter files" % kernel)
    copied = 512 * 1024  # KiB
    ff, fw = copied / copy_f, copied / copy_w
    fetch_b = sum(kf) / len(kf) * 1024 * ff
    write_b = sum(kw) / len(kw) * 1024 * fw
    h = hashlib.sha256()
    for f in source.split(","):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    h = h.hexdigest()[:16]
    out = ["# HBM traffic counters: %s, %s workload" % (kernel, workload), "",
           "Commands (one counter per run; bench.py ends with one 512 MiB device copy for calibration):", "",
           "    " + cmd_fetch, "    " + cmd_write, "",
           "Then `python profile_summary.py traffic <fetch dir> <write dir> %s %s '%s' %s`." % (tag, workload, kernel, source), "",
           "| quantity | value |", "|---|---|",
           "| calibration copy: FETCH_SIZE KiB read for 524288 KiB copied | %.1f (factor %.3f) |" % (copy_f, ff),
           "| calibration copy: WRITE_SIZE KiB for 524288 KiB copied | %.1f (factor %.3f) |" % (copy_w, fw),
           "| dominant kernel launches sampled | %d (fetch), %d (write) |" % (len(kf), len(kw)),
           "| FETCH_SIZE per launch, raw KiB | %.1f |" % (sum(kf) / len(kf)),
           "| WRITE_SIZE per launch, raw KiB | %.1f |" % (sum(kw) / len(kw)),
           "| HBM bytes read per launch (scaled) | %.4g |" % fetch_b,
           "| HBM bytes written per launch (scaled) | %.4g |" % write_b,
           "| HBM bytes per launch (scaled) | %.4g |" % (fetch_b + write_b),
           "| sha256 (first 16 hex) of %s when taken | %s |" % (", ".join(os.path.basename(f) for f in source.split(",")), h)]
    text = "\n".join(out) + "\n"
    open(os.path.join(PROFILES, "%s_traffic.md" % tag), "w").write(text)
    tj = os.path.join(PROFILES, "traffic.json")
    d = json.load(open(tj)) if os.path.exists(tj) else {}
    d[workload] = dict(kernel=kernel, bytes_per_launch=fetch_b + write_b, read_bytes=fetch_b,
                       write_bytes=write_b, fetch_factor=ff, write_factor=fw,
                       gemm_source_sha256_16=h, summary="%s_traffic.md" % tag)
    json.dump(d, open(tj, "w"), indent=1)
    return text


def bench(run_dir: str) -> str:
    rows, raw = [], []
    for path in sorted(glob.glob(os.path.join(run_dir, "*.json"))):
        name = os.path.splitext(os.path.basename(path))[0]
        lines = [l for l in open(path).read().splitlines() if l.startswith("{")]
        if not lines:
            continue
        d = json.loads(lines[-1])
        cmd = open(os.path.join(run_dir, name + ".cmd")).read().strip()
        st = d.get("step_ms") or {}
        rf = d.get("roofline") or {}
        rows.append("| %s | `%s` | %.6g %s | %s | %s | %s | %s |" % (
            name, cmd, d["value"], d["unit"],
            "%.4g / %.4g / %.4g" % (st["median"], st["p10"], st["p90"]) if st else "%.4g" % d["ms_per_step"],
            ("%s: %.3g %s (%.1f %%)" % (rf.get("kernel", ""), rf["achieved"], rf["unit"], 100 * rf["frac"])) if rf else "",
            ("%.4g" % rf["traffic"]) if rf.get("traffic") else "null",
            d.get("config", {}).get("workload", "")))
        raw.append("    " + lines[-1])
    out = ["# bench.py lines, one MI355X", "",
           "Each row is one run of the command shown, from the repository root; the table gives the",
           "headline value, the step time in ms (median / p10 / p90 over the timed steps), the dominant",
           "kernel's roofline figure and its measured HBM bytes per launch (`traffic`, null when no",
           "counter summary matches the current kernel source). The full JSON lines follow.", "",
           "Then `python profile_summary.py bench <run dir>`.", "",
           "| run | command | value | step ms (median / p10 / p90) | dominant kernel | traffic B | workload |",
           "|---|---|---|---|---|---|---|"] + rows + ["", "Full lines:", ""] + raw
    text = "\n".join(out) + "\n"
    open(os.path.join(PROFILES, "bench_lines.md"), "w").write(text)
    return text


def counters(tag: str, kernel: str, dirs, cmd: str) -> str:
    vals = {}
    for d in dirs:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))):
            if kernel in r["Kernel_Name"]:
                per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for name, by_dispatch in per.items():
            vals[name] = (statistics.mean(by_dispatch.values()), len(by_dispatch))
    if not vals:
        raise SystemExit("kernel %r not found in the counter files" % kernel)
    out = ["# SQ counters: %s" % kernel, "", "Command (one pass per counter set, from the repository root):", "",
           "    " + cmd, "", "Then `python profile_summary.py counters %s '%s' <run dirs>`." % (tag, kernel), "",
           "Values are per launch (average over the launches sampled), summed over the hardware",
           "instances that report them.", "",
           "| counter | per launch | launches |", "|---|---|---|"]
    for name in sorted(vals):
        out.append("| %s | %.4g | %d |" % (name, vals[name][0], vals[name][1]))
    v = {k: x[0] for k, x in vals.items()}
    ratios = []
    if "SQ_VALU_MFMA_BUSY_CYCLES" in v and "SQ_BUSY_CU_CYCLES" in v:
        ratios.append(("MFMA pipes busy, share of SIMD cycles (MFMA_BUSY / (4 BUSY_CU))",
                       v["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * v["SQ_BUSY_CU_CYCLES"])))
    if "SQ_INSTS_MFMA" in v:
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS"):
            if k in v:
                label = "VALU (MFMA included)" if k == "SQ_INSTS_VALU" else k[9:]
                ratios.append(("%s instructions per MFMA instruction" % label, v[k] / v["SQ_INSTS_MFMA"]))
    if "SQ_LDS_BANK_CONFLICT" in v and "SQ_INSTS_LDS" in v:
        ratios.append(("LDS bank-conflict cycles per LDS instruction", v["SQ_LDS_BANK_CONFLICT"] / v["SQ_INSTS_LDS"]))
    if "SQ_WAIT_INST_ANY" in v and "SQ_WAVE_CYCLES" in v:
        ratios.append(("wave cycles waiting to issue, share (WAIT_INST_ANY / WAVE_CYCLES)", v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"]))
    if "SQ_WAIT_INST_LDS" in v and "SQ_WAVE_CYCLES" in v:
        ratios.append(("wave cycles waiting to issue an LDS instruction, share", v["SQ_WAIT_INST_LDS"] / v["SQ_WAVE_CYCLES"]))
    if ratios:
        out += ["", "| derived | value |", "|---|---|"] + ["| %s | %.3f |" % r for r in ratios]
    text = "\n".join(out) + "\n"
    open(os.path.join(PROFILES, "%s_counters.md" % tag), "w").write(text)
    return text


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("run_dir")
    k.add_argument("tag")
    k.add_argument("--last", type=int, required=True)
    k.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    for a in ("fetch_dir", "write_dir", "tag", "workload", "kernel", "source"):
        t.add_argument(a)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    b = sub.add_parser("bench")
    b.add_argument("run_dir")
    c = sub.add_parser("counters")
    c.add_argument("tag")
    c.add_argument("kernel")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.what == "bench":
        print(bench(a.run_dir))
    elif a.what == "counters":
        print(counters(a.tag, a.kernel, a.dirs, a.cmd))
    elif a.what == "kernels":
        print(kernels(a.run_dir, a.tag, a.last, a.cmd))
    else:
        print(traffic(a.fetch_dir, a.write_dir, a.tag, a.workload, a.kernel, a.source, a.cmd_fetch,
                      a.cmd_write))


if __name__ == "__main__":
    main()
