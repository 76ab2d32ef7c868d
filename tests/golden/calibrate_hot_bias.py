"""Find the router bias of the skewed 4-bit prefill workload's hot set.

The workload (8192 tokens, hidden 4096, 256 experts, top-8) asks for 10 % of the experts to
receive 50 % of all assignments.  This script bisects the constant bias added to the hot
experts' logits until the realised share, computed by the CPU oracle's routing on the seeded
tokens, is 0.50 +- 0.005, and prints the value to freeze in ``synth.HOT_BIAS``.

Run:  python tests/golden/calibrate_hot_bias.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))

from mixture_experts_layer_softmax_amd import synth  # noqa: E402
from oracle import oracle  # noqa: E402


def hot_share(inputs, wl, beta):
    b = synth.router_bias(wl, hot_bias=beta)
    logits = oracle.router_logits(inputs["x"], inputs["w_router"], b)
    ids, _ = oracle.select(logits, wl.top_k)
    return float(np.isin(ids, synth.hot_set(wl)).mean())


def main():
    wl = synth.WORKLOADS["nvfp4_prefill"]
    inputs = synth.generate(wl, with_experts=False)
    lo, hi = 0.0, 8.0
    for _ in range(40):
        mid = np.float32((lo + hi) / 2)
        s = hot_share(inputs, wl, float(mid))
        print("beta %.6f share %.5f" % (mid, s), flush=True)
        if abs(s - synth.HOT_SHARE_TARGET) <= 0.001:
            break
        lo, hi = (float(mid), hi) if s < synth.HOT_SHARE_TARGET else (lo, float(mid))
    # round to a short decimal that still meets the target
    for digits in (2, 3, 4, 5, 6):
        r = float(np.float32(round(float(mid), digits)))
        if abs(hot_share(inputs, wl, r) - synth.HOT_SHARE_TARGET) <= 0.005:
            print("HOT_BIAS =", r)
            return r
    print("HOT_BIAS =", float(mid))
    return float(mid)


if __name__ == "__main__":
    main()
