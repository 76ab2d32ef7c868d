"""moe_forward_static (the entry point for callers that cannot allocate) against moe_forward
with a caller workspace, through the C ABI: bit-identical outputs and routing, on two calls in
a row with a smaller batch the second time (the static scratch keeps the first call's contents),
for bf16, NVFP4 and fp32 layers; a problem larger than the scratch is refused before any device
work."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_softmax_amd import lib, synth
from mixture_experts_layer_softmax_amd.layer import MoELayer

pytestmark = pytest.mark.gpu


def note(msg):
    print("[gpu] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _env():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib.load()


def _debug(layer, T):
    dev, k, E = layer.device, layer.k, layer.E
    return dict(topk_ids=torch.empty(T, k, dtype=torch.int32, device=dev),
                topk_w=torch.empty(T, k, dtype=torch.float32, device=dev),
                counts=torch.empty(E, dtype=torch.int32, device=dev),
                offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                sorted_token=torch.empty(T * k, dtype=torch.int32, device=dev),
                inv_perm=torch.empty(T * k, dtype=torch.int32, device=dev))


@pytest.mark.parametrize("name,first,second", [("decode64", 64, 5), ("nvfp4_decode", 16, 3),
                                               ("tiny", 64, 7)])
def test_static_scratch_forward_equals_workspace_forward(name, first, second):
    wl = synth.WORKLOADS[name]
    inp = synth.generate(wl.with_tokens(first, x_sub=900 + first))
    layer = MoELayer.from_workload(wl.with_tokens(first), inp)
    x_all = layer.act_tensor(inp["x"])
    for T in (first, second):
        note("%s: moe_forward_static vs moe_forward, T=%d" % (name, T))
        x = x_all[:T].contiguous()
        p = layer.problem_for(T)
        ws = torch.empty(lib.workspace_size(p), dtype=torch.uint8, device=layer.device)
        assert lib.workspace_size(p) <= lib.STATIC_SCRATCH_BYTES
        y_ref = layer.empty_act(T, wl.hidden)
        d_ref = _debug(layer, T)
        lib.forward(p, x, layer.w_router, layer.bias, layer.weights, y_ref, ws, **d_ref)
        y = layer.empty_act(T, wl.hidden)
        d = _debug(layer, T)
        lib.forward_static(p, x, layer.w_router, layer.bias, layer.weights, y, **d)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.uint8), y_ref.view(torch.uint8))
        for key in d:
            assert torch.equal(d[key], d_ref[key]), key


def test_static_scratch_refuses_a_problem_larger_than_it():
    wl = synth.WORKLOADS["prefill"]
    p = lib.problem(wl.tokens, wl.hidden, wl.experts, wl.top_k, wl.ffn)
    assert lib.workspace_size(p) > lib.STATIC_SCRATCH_BYTES
    fake = torch.empty(16, dtype=torch.uint8, device="cuda")  # never dereferenced: refused first
    w = lib.weights(fake, fake, layout=lib.LAYOUT_PACKED)
    with pytest.raises(lib.MoeError) as err:
        lib.forward_static(p, fake, fake, None, w, fake)
    assert err.value.status == lib.MOE_ERR_SCRATCH_TOO_SMALL
    note("prefill-sized problem refused: %s" % lib.status_string(err.value.status))
