"""GPU parity of the MX layers (MXFP8 and MXFP4 weights, MXFP8 activations, block-scaled
matrix cores) against the CPU oracle.

The activation quantizer is an integer decision on exact bf16 inputs, so its codes and scales
must match the oracle's bit for bit.  Both sides quantize the same activations: x is bf16, and
hid, the layer's bf16 activation between the two projections, is rounded to bf16 before it is
quantized (the oracle rounds its fp64 hid to bf16 first; a CPU pin with a hand-worked block
checks that reading).  The layer outputs are held to the same 2e-2 max relative error as every
other format: the GPU's hid differs from the oracle's by its fp32 accumulation order, which can
move a bf16 rounding and then an E4M3 rounding by one step for a few elements.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_softmax_amd import lib, synth
from mixture_experts_layer_softmax_amd.layer import MoELayer, bf16_bits_to_f64, to_device, to_host
from gpu_checks import check_experts_through_stages, p99_err
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2
W = synth.Workload
SMALL = {}
for _wdt in ("mxfp8", "mxfp4"):
    SMALL.update({
        "small_" + _wdt: W("small_" + _wdt, 384, 512, 16, 4, 512, "bf16", _wdt, 17, "normal"),
        "ragged_" + _wdt: W("ragged_" + _wdt, 77, 1024, 5, 3, 1536, "bf16", _wdt, 18, "normal"),
        "one_token_" + _wdt: W("one_token_" + _wdt, 1, 512, 8, 2, 512, "bf16", _wdt, 19, "none"),
        # K = 2048 on both GEMMs and few rows: the decode kernel splits K over 4 wavefronts
        "split_" + _wdt: W("split_" + _wdt, 4, 2048, 8, 2, 2048, "bf16", _wdt, 20, "normal"),
    })


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


def test_quantizer_matches_oracle_bit_exactly():
    rng = np.random.default_rng(41)
    rows, K = 640, 512
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (rows, 1))).astype(np.float32)  # row-wise magnitudes
    x[0] = 0.0                                                        # all-zero blocks
    x[1, :32] = -0.0
    x[2] = rng.standard_normal(K).astype(np.float32) * 1e-38          # bf16 subnormals
    x[3] = rng.standard_normal(K).astype(np.float32) * 1e30           # large exponents
    x[4] = (rng.integers(0, 33, K) * 2 + 1).astype(np.float32) / 64   # many E4M3 rounding ties
    x[5, ::32] = 450.0                                                # clamped block maxima
    bits = synth.to_bf16_bits(x)
    ref_c, ref_s, _ = O.mx_quantize(bits)
    xd = to_device(bits, "cuda")
    codes = torch.empty(rows, K, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, K // 32, dtype=torch.uint8, device="cuda")
    note("mx quantize %dx%d" % (rows, K))
    lib.quantize_mxfp8(xd, codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def _check_forward(wl, inp, layer, tokens=None):
    x = layer.act_tensor(inp["x"])
    y, dbg = layer.forward(x, debug=True)
    torch.cuda.synchronize()
    ref = O.forward(inp, wl.top_k, wl.wdt, wl.ffn, wl.renormalize, tokens=tokens)
    for key in ("topk_ids", "counts", "offsets", "sorted_token", "inv_perm"):
        got = dbg[key].cpu().numpy()
        assert np.array_equal(got.reshape(ref[key].shape), ref[key]), key
    got = bf16_bits_to_f64(to_host(y))[ref["tokens"]]
    e = rel_err(got, ref["y"])
    note("  %s y rel err %.3e, per-element p99 %.3e, over %d tokens"
         % (wl.name, e, p99_err(got, ref["y"]), len(ref["tokens"])))
    assert e <= TOL


@pytest.mark.parametrize("path", ["prefill", "decode"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_forward_matches_oracle(name, path):
    wl = SMALL[name]
    inp = synth.generate(wl)
    note("MX forward %s path=%s" % (name, path))
    _check_forward(wl, inp, MoELayer.from_workload(wl, inp, path=path))


@pytest.mark.parametrize("path", ["prefill", "decode"])
@pytest.mark.parametrize("wdt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("kind", [lib.GATE_UP_SWIGLU, lib.DOWN])
def test_grouped_gemm_matches_oracle(kind, wdt, path):
    wl = SMALL["small_" + wdt]
    inp = synth.generate(wl)
    layer = MoELayer.from_workload(wl, inp, path=path)
    r = O.route(inp, wl.top_k)
    A = wl.assignments
    expert_of_row = np.searchsorted(r["offsets"], np.arange(A), side="right") - 1
    p = layer.problem_for(wl.tokens)
    ws = layer.workspace(wl.tokens)
    offsets = torch.from_numpy(r["offsets"]).cuda()
    note("%s grouped gemm kind %d" % (wdt, kind))
    if kind == lib.GATE_UP_SWIGLU:
        out = layer.empty_act(A, wl.ffn)
        lib.grouped_gemm(p, kind, layer.act_tensor(inp["x"]), torch.from_numpy(r["sorted_token"]).cuda(),
                         offsets, layer.weights, out, ws)
        ref = O.gate_up_rows(inp, wdt, wl.ffn, r["sorted_token"], expert_of_row)
    else:
        hid = synth.to_bf16_bits(np.random.default_rng(3).standard_normal((A, wl.ffn)).astype(np.float32) * 0.05)
        out = layer.empty_act(A, wl.hidden)
        lib.grouped_gemm(p, kind, to_device(hid, "cuda"), None, offsets, layer.weights, out, ws)
        ref = O.down_rows(inp, wdt, wl.hidden, bf16_bits_to_f64(hid), expert_of_row)
    torch.cuda.synchronize()
    e = rel_err(bf16_bits_to_f64(to_host(out)), ref)
    note("  rel err %.3e" % e)
    assert e <= TOL


@pytest.mark.parametrize("path", ["prefill", "decode"])
@pytest.mark.parametrize("wdt", ["mxfp8", "mxfp4"])
def test_expert_parallel_share(wdt, path):
    wl = SMALL["small_" + wdt]
    b, n = 4, 8
    inp = synth.generate(wl, experts=range(b, b + n))
    layer = MoELayer.from_workload(wl, inp, path=path, expert_begin=b, local_experts=n)
    x = layer.act_tensor(inp["x"])
    y, dbg = layer.forward(x, debug=True)
    torch.cuda.synchronize()
    ref = O.forward(inp, wl.top_k, wl.wdt, wl.ffn, held=(b, n))
    assert np.array_equal(dbg["inv_perm"].cpu().numpy().reshape(ref["inv_perm"].shape), ref["inv_perm"])
    e = rel_err(bf16_bits_to_f64(to_host(y)), ref["y"])
    note("  %s share [%d, %d): y rel err %.3e" % (wdt, b, b + n, e))
    assert e <= TOL


@pytest.mark.parametrize("layout", ["packed", "row_major"])
@pytest.mark.parametrize("wdt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_down_with_one_hot_rows_returns_exact_weights(wdt, path, layout):
    """hid row r = unit vector at f_r: its MXFP8 form is exact (scale 2^-8, code 256), so
    y_perm[r, h] must equal the decoded weight W2[e][h, f_r] exactly (an E4M3 or E2M1 value
    times a power of two, exact in bf16); this pins the weight layout, the chunk slots and the
    scale bytes of both MX kernels."""
    E, H, F = 3, 512, 512
    wl = W("onehot_" + wdt, 1, H, E, 1, F, "bf16", wdt, 23, "none")
    inp = synth.generate(wl)
    A = E * F
    f_of_row = np.tile(np.arange(F), E)
    e_of_row = np.repeat(np.arange(E), F).astype(np.int32)
    hid = np.zeros((A, F), np.float32)
    hid[np.arange(A), f_of_row] = 1.0
    hid_bits = synth.to_bf16_bits(hid)
    ref = O.down_rows(inp, wdt, H, bf16_bits_to_f64(hid_bits), e_of_row)
    layer = MoELayer(A, H, E, 1, F, "bf16", wdt, inp, path=path, weight_layout=layout)
    p = layer.problem_for(A)
    ws = layer.workspace(A)
    y_perm = layer.empty_act(A, H)
    offsets = np.arange(E + 1, dtype=np.int32) * F
    note("MX one-hot down wdt=%s path=%s layout=%s" % (wdt, path, layout))
    lib.grouped_gemm(p, lib.DOWN, to_device(hid_bits, "cuda"), None, torch.from_numpy(offsets).cuda(),
                     layer.weights, y_perm, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_to_f64(to_host(y_perm)), ref)


@pytest.mark.parametrize("name", ["mxfp8_prefill", "mxfp4_prefill"])
def test_full_size_prefill(name):
    """Routing bit-exact on every token, the output on sampled tokens, and every hid and y_perm
    row of three whole experts through the stage entry points (gpu_checks)."""
    wl = synth.WORKLOADS[name]
    note("%s: generating inputs" % name)
    inp = synth.generate(wl)
    layer = MoELayer.from_workload(wl, inp)
    rng = np.random.default_rng(98)
    toks = np.unique(np.concatenate([[0, wl.tokens - 1], rng.choice(wl.tokens, 10, replace=False)]))
    note("%s: running" % name)
    _check_forward(wl, inp, layer, tokens=toks)
    note("%s: stage entry points, whole experts" % name)
    check_experts_through_stages(wl, inp, layer, note)


@pytest.mark.parametrize("name", ["mxfp8_decode64", "mxfp4_decode64"])
def test_decode64_every_token(name):
    wl = synth.WORKLOADS[name]
    note("%s: generating inputs" % name)
    inp = synth.generate(wl)
    note("%s: all 64 tokens" % name)
    _check_forward(wl, inp, MoELayer.from_workload(wl, inp))


@pytest.mark.parametrize("wdt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_row_major_codes_give_the_packed_layer(wdt, path):
    """MX codes handed over row-major give the packed layer bit for bit."""
    wl = SMALL["ragged_" + wdt]
    inp = synth.generate(wl)
    a = MoELayer.from_workload(wl, inp, path=path)
    b = MoELayer.from_workload(wl, inp, path=path, weight_layout="row_major")
    assert a.layout == lib.LAYOUT_PACKED and b.layout == lib.LAYOUT_ROW_MAJOR
    x = a.act_tensor(inp["x"])
    note("MX row-major codes %s path=%s" % (wdt, path))
    ya = a.forward(x).clone()
    yb = b.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)
