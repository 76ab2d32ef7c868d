"""moe_forward captured in a HIP graph replays to the same bits as eager calls.

The forward only launches kernels onto the caller's stream: no allocation, no memset, no
synchronisation and no read-back to the host (grids are sized from host-side bounds and the
kernels read the tile counts on the device).  A caller may therefore capture it once and
replay it.  Each case captures one forward on a static input, then replays it for two token
sets in turn (the second one negated, so the routing, the tile lists and the grid occupancy
differ between replays), with eager forwards and synchronisations between the replays, and
compares every replay bit for bit with an eager forward of the same tokens.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_softmax_amd import lib, synth
from mixture_experts_layer_softmax_amd.layer import MoELayer

pytestmark = pytest.mark.gpu

W = synth.Workload
CASES = {
    # workload, path (None: the library's choice for the batch size)
    "decode1": (synth.WORKLOADS["decode1"], None),
    "decode8": (synth.WORKLOADS["decode8"], None),
    "nvfp4_decode": (synth.WORKLOADS["nvfp4_decode"], None),
    "tiny": (synth.WORKLOADS["tiny"], None),
    "small_bf16_prefill": (W("small_bf16", 512, 512, 8, 2, 256, "bf16", "bf16", 11, "normal"), "prefill"),
    "small_nvfp4_prefill": (W("small_nvfp4", 384, 512, 16, 4, 256, "bf16", "nvfp4", 12, "normal"), "prefill"),
    "small_mxfp8": (W("small_mxfp8", 96, 512, 16, 4, 512, "bf16", "mxfp8", 17, "normal"), None),
    "small_mxfp4_decode": (W("small_mxfp4", 24, 512, 16, 4, 512, "bf16", "mxfp4", 17, "normal"), "decode"),
}


def note(msg):
    print("[gpu] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _env():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib.load()


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager_forwards(name):
    wl, path = CASES[name]
    T = wl.tokens
    inp = synth.generate(wl)
    layer = MoELayer.from_workload(wl, inp, path=path or "auto")
    xa = layer.act_tensor(inp["x"])
    xb = -torch.flip(xa, [0])  # exact in bf16 and fp32; changes which experts are picked
    x = xa.clone()
    y = layer.empty_act(T, wl.hidden)
    note("graph %s: T=%d, warm-up" % (name, T))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, y=y, path=path)  # sizes the workspace outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph %s: capture" % name)
    with torch.cuda.graph(g):
        layer.forward(x, y=y, path=path)
    torch.cuda.synchronize()
    routes = set()
    for rep, src in enumerate([xa, xb, xa, xb]):
        x.copy_(src)
        note("graph %s: replay %d" % (name, rep))
        g.replay()
        got = y.clone()
        ref, dbg = layer.forward(src.clone(), debug=True, path=path)
        torch.cuda.synchronize()
        routes.add(tuple(dbg["topk_ids"].flatten().tolist()))
        assert torch.equal(_bits(got), _bits(ref)), "replay %d differs from the eager forward" % rep
        assert bool(torch.isfinite(got.float()).all())
    assert len(routes) == 2, "the two token sets should route differently"
