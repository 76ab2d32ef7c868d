"""The single-launch decode kernel (MOE_PATH_DECODE_FUSED) against the multi-launch decode path
and the CPU oracle.

Both paths run the same device code in the same order: routing and dispatch must be bit-equal,
the layer output within the 2e-2 bar of the oracle, and bit-equal to the multi-launch output
where both split K the same way.  The grid barriers are checked for completing without a
time-out, for counting time-outs instead of hanging when the host forces a spin limit of zero,
and timed on their own by the barrier probe.
"""
import os
import time

import numpy as np
import pytest
import torch

from mixture_experts_layer_softmax_amd import lib, synth
from mixture_experts_layer_softmax_amd.layer import MoELayer, bf16_bits_to_f64, to_host
from gpu_checks import p99_err
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2
W = synth.Workload
ROUTING = ("topk_ids", "topk_w", "counts", "offsets", "sorted_token", "inv_perm")


def note(msg):
    print("[gpu] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _env():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib.load()
    O.build()


def rel_err(y, ref):
    return float(np.max(np.abs(y - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def timeouts(layer):
    """The count of barrier waits that gave up, at byte offset 8 of the workspace."""
    return int(layer.ws[8:12].view(torch.int32).item())


CASES = {
    "decode1": (synth.WORKLOADS["decode1"], "packed"),
    "decode8": (synth.WORKLOADS["decode8"], "packed"),
    "decode1_rm": (synth.WORKLOADS["decode1"], "row_major"),
    "nvfp4_decode": (synth.WORKLOADS["nvfp4_decode"], "packed"),
    "nvfp4_decode_t3": (synth.WORKLOADS["nvfp4_decode"].with_tokens(3, x_sub=3), "packed"),
    # k = 16 over 64 experts: 256 dispatched rows, the kernel's largest batch
    "k16": (W("k16", 16, 512, 64, 16, 512, "bf16", "bf16", 81, "normal"), "packed"),
    "renorm0": (W("renorm0", 5, 512, 32, 4, 512, "bf16", "bf16", 82, "normal", renormalize=False), "packed"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_decode_matches_oracle_and_multi_launch(name):
    wl, layout = CASES[name]
    inp = synth.generate(wl)
    layer = MoELayer.from_workload(wl, inp, weight_layout=layout)
    x = layer.act_tensor(inp["x"])
    note("fused decode %s T=%d E=%d k=%d" % (name, wl.tokens, wl.experts, wl.top_k))
    y_d, d_d = layer.forward(x, debug=True, path="decode")
    y_d = y_d.clone()
    layer.ws.zero_()  # barrier words: the time-out count starts at zero
    y_f, d_f = layer.forward(x, debug=True, path="fused")
    y_f2 = layer.forward(x, path="fused").clone()  # a second call: the sequence number moved on
    torch.cuda.synchronize()
    assert timeouts(layer) == 0
    for key in ROUTING:
        assert torch.equal(d_f[key], d_d[key]), key
    assert torch.equal(y_f, y_f2)
    ref = O.forward(inp, wl.top_k, wl.wdt, wl.ffn, wl.renormalize)
    got = bf16_bits_to_f64(to_host(y_f))
    e = rel_err(got, ref["y"])
    e_ml = rel_err(got, bf16_bits_to_f64(to_host(y_d)))
    note("  y rel err %.3e (per-element p99 %.3e) vs oracle, %.3e vs the multi-launch path"
         % (e, p99_err(got, ref["y"]), e_ml))
    assert e <= TOL
    if wl.tokens == 1 and wl.wdt == "bf16":  # both paths split K four ways here
        assert torch.equal(y_f, y_d)


def test_fused_decode_held_expert_range():
    wl = synth.WORKLOADS["decode8"]
    b, n = 32, 64
    inp = synth.generate(wl, experts=range(b, b + n))
    layer = MoELayer.from_workload(wl, inp, expert_begin=b, local_experts=n)
    x = layer.act_tensor(inp["x"])
    note("fused decode, experts [%d, %d)" % (b, b + n))
    y_d = layer.forward(x, path="decode").clone()
    y_f, d_f = layer.forward(x, debug=True, path="fused")
    torch.cuda.synchronize()
    ref = O.forward(inp, wl.top_k, wl.wdt, wl.ffn, held=(b, n))
    assert np.array_equal(d_f["inv_perm"].cpu().numpy().reshape(ref["inv_perm"].shape), ref["inv_perm"])
    assert rel_err(bf16_bits_to_f64(to_host(y_f)), ref["y"]) <= TOL
    assert rel_err(bf16_bits_to_f64(to_host(y_f)), bf16_bits_to_f64(to_host(y_d))) <= 1e-2


def test_fused_decode_rejects_what_it_does_not_cover():
    wl = synth.WORKLOADS["decode64"]  # 64 tokens: more than the kernel's 16
    inp = synth.generate(wl)
    layer = MoELayer.from_workload(wl, inp)
    with pytest.raises(lib.MoeError) as err:
        layer.forward(layer.act_tensor(inp["x"]), path="fused")
    assert err.value.status == lib.MOE_ERR_UNSUPPORTED


def test_barrier_time_outs_are_counted_instead_of_hanging():
    """A spin limit of zero (forced from the host) makes barrier waits give up at their first
    unsuccessful poll: the launch still completes and the count is non-zero; the next call with
    the default limit completes without a time-out and gives the layer again."""
    wl = synth.WORKLOADS["decode1"]
    inp = synth.generate(wl)
    layer = MoELayer.from_workload(wl, inp)
    x = layer.act_tensor(inp["x"])
    y_ref = layer.forward(x, path="decode").clone()
    layer.ws.zero_()
    os.environ["MOE_FUSED_SPIN_LIMIT"] = "0"
    try:
        note("fused decode with spin limit 0")
        layer.forward(x, path="fused")
        torch.cuda.synchronize()
    finally:
        del os.environ["MOE_FUSED_SPIN_LIMIT"]
    n = timeouts(layer)
    note("  %d barrier waits gave up" % n)
    assert n > 0
    layer.ws.zero_()
    y = layer.forward(x, path="fused")
    torch.cuda.synchronize()
    assert timeouts(layer) == 0
    assert torch.equal(y, y_ref)


@pytest.mark.parametrize("blocks", [256, 1024])
def test_barrier_probe_cost(blocks):
    """Time one grid barrier at the decode kernel's grid sizes (printed; bounded for sanity)."""
    sync = torch.zeros(lib.PROBE_SYNC_BYTES, dtype=torch.uint8, device="cuda")
    lib.probe_grid_barrier(blocks, 10, sync)
    torch.cuda.synchronize()
    n = 2000
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    lib.probe_grid_barrier(blocks, n, sync)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n
    note("grid barrier over %d blocks: %.2f us" % (blocks, us))
    assert int(sync[8:12].view(torch.int32).item()) == 0
    assert us < 100.0
