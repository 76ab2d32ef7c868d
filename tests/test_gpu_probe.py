"""The measurement probes of moe_probe.h run and report plausible rates (sanity, not parity)."""
import pytest
import torch

from mixture_experts_layer_softmax_amd import lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _env():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib.load()


def _rate(fn):
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    work = fn()
    b.record()
    torch.cuda.synchronize()
    return work / (a.elapsed_time(b) * 1e-3)


def test_mfma_probe_rate_is_plausible():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.full((8 * cus,), -1.0, dtype=torch.float32, device="cuda")
    r = _rate(lambda: lib.probe_mfma_bf16(8 * cus, 2000, sink))
    print("[gpu] mfma probe %.1f TFLOP/s" % (r / 1e12), flush=True)
    assert torch.isfinite(sink).all() and (sink != -1.0).all()
    assert 2e14 < r < 3.0e15  # between 8 % and 120 % of the 2.5 PFLOP/s data-sheet peak


@pytest.mark.parametrize("nontemporal", [False, True])
def test_read_probe_rate_is_plausible(nontemporal):
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    r = _rate(lambda: lib.probe_read(buf, word, nontemporal=nontemporal))
    print("[gpu] read probe (nontemporal=%s) %.1f GB/s" % (nontemporal, r / 1e9), flush=True)
    assert 1e12 < r < 1.2e13


@pytest.mark.parametrize("wdt", ["bf16", "nvfp4"])
def test_grouped_gemm_timing_probe_runs_the_same_gemm(wdt):
    """moe_probe_grouped_gemm_times writes what moe_grouped_gemm writes (bit for bit) and
    returns one positive time per launch, no longer than a whole moe_grouped_gemm call."""
    from mixture_experts_layer_softmax_amd import synth
    from mixture_experts_layer_softmax_amd.layer import MoELayer

    wl = synth.Workload("probe_" + wdt, 512, 512, 16, 4, 256, "bf16", wdt, 77, "none")
    inp = synth.generate(wl)
    layer = MoELayer.from_workload(wl, inp)
    x = layer.act_tensor(inp["x"])
    y, dbg = layer.forward(x, debug=True)
    p = layer.problem_for(wl.tokens)
    ws = layer.workspace(wl.tokens)
    hid = layer.empty_act(wl.assignments, wl.ffn)
    hid2 = layer.empty_act(wl.assignments, wl.ffn)
    print("[gpu] timing probe, %s weights" % wdt, flush=True)
    lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x, dbg["sorted_token"], dbg["offsets"], layer.weights, hid, ws)
    flush = torch.ones(1 << 26, dtype=torch.uint8, device="cuda")
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    for fb in (None, flush):
        hid2.zero_()
        ms = lib.probe_grouped_gemm_times(p, lib.GATE_UP_SWIGLU, x, dbg["sorted_token"], dbg["offsets"],
                                          layer.weights, hid2, ws, 5, flush=fb, flush_out=word)
        torch.cuda.synchronize()
        assert torch.equal(hid.view(torch.int16), hid2.view(torch.int16))
        assert len(ms) == 5 and all(0.0 < t < 1000.0 for t in ms)
        print("[gpu]   flush=%s: %s ms" % (fb is not None, ", ".join("%.4f" % t for t in ms)), flush=True)
