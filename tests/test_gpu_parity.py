"""GPU parity: every C-ABI entry point against the CPU oracle on seeded inputs.

Bar: expert ids, counts, offsets, sorted_token and inv_perm bit-exact; routing weights within
1e-5 relative; layer outputs within 2e-2 max relative error (max|y - ref| / max|ref|).
Small shapes run the oracle on everything; the full-size workloads check routing and dispatch
on every token, the layer output on a sample of tokens (all 64 in the 64-token decode batch),
and every row of three whole experts through the stage entry points.
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
W_RTOL = 1e-5
W = synth.Workload

# small shapes spanning several row tiles with ragged tails and skewed expert loads
SMALL = {
    "small_bf16": W("small_bf16", 512, 512, 8, 2, 256, "bf16", "bf16", 11, "normal"),
    "small_nvfp4": W("small_nvfp4", 384, 512, 16, 4, 256, "bf16", "nvfp4", 12, "normal"),
    "ragged_bf16": W("ragged_bf16", 77, 256, 5, 3, 384, "bf16", "bf16", 13, "normal"),
    "ragged_nvfp4": W("ragged_nvfp4", 77, 192, 5, 3, 320, "bf16", "nvfp4", 14, "normal"),
    # K = 2048 on both GEMMs: the NVFP4 decode kernel takes its 512-wide scale windows
    "win4_nvfp4": W("win4_nvfp4", 8, 2048, 16, 2, 2048, "bf16", "nvfp4", 15, "normal"),
    "ragged_f32": W("ragged_f32", 33, 128, 5, 2, 192, "f32", "f32", 16, "normal"),
    "tiny": synth.WORKLOADS["tiny"],
    # top-16 routing with F = 128 (one token: 16 slots through the single-block dispatch)
    "k16_bf16": W("k16_bf16", 64, 512, 32, 16, 128, "bf16", "bf16", 41, "normal"),
    # MX layers: the forward's gate/up epilogue writes hid as MXFP8 itself
    "small_mxfp8": W("small_mxfp8", 384, 512, 16, 4, 512, "bf16", "mxfp8", 17, "normal"),
    "small_mxfp4": W("small_mxfp4", 384, 512, 16, 4, 512, "bf16", "mxfp4", 17, "normal"),
    "split_mxfp8": W("split_mxfp8", 4, 2048, 8, 2, 2048, "bf16", "mxfp8", 20, "normal"),
}


def note(msg):
    print("[gpu] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _env():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib.load()
    O.build()


_CACHE = {}


def case(name):
    """Workload of a case name; a name ending in _rm hands the weights over row-major (the other
    cases pack bf16 and MX weights, and NVFP4 weights wherever the shape allows it)."""
    rm = name.endswith("_rm")
    base = name[:-3] if rm else name
    return SMALL.get(base) or synth.WORKLOADS[base], ("row_major" if rm else "packed")


def inputs_of(wl):
    key = (wl.name, wl.tokens, wl.x_sub)
    if key not in _CACHE:
        _CACHE.clear()
        _CACHE[key] = synth.generate(wl)
    return _CACHE[key]


def act_f64(a):
    return a.astype(np.float64) if a.dtype == np.float32 else bf16_bits_to_f64(a)


def rel_err(y, ref):
    return float(np.max(np.abs(y - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


# ---------------------------------------------------------------------------------------
# route
# ---------------------------------------------------------------------------------------

ROUTE_CASES = ["tiny", "small_bf16", "small_nvfp4", "ragged_bf16", "decode1", "decode8",
               "decode64", "nvfp4_decode", "prefill", "nvfp4_prefill"]


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_matches_oracle(name):
    wl = SMALL.get(name) or synth.WORKLOADS[name]
    inp = synth.generate(wl, with_experts=False)
    note("route %s T=%d E=%d k=%d" % (name, wl.tokens, wl.experts, wl.top_k))
    ref = O.route(inp, wl.top_k)
    p = lib.problem(wl.tokens, wl.hidden, wl.experts, wl.top_k, wl.ffn, wl.act, wl.wdt)
    ws = torch.empty(lib.workspace_size(p), dtype=torch.uint8, device="cuda")
    ids = torch.empty(wl.tokens, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(wl.tokens, wl.top_k, dtype=torch.float32, device="cuda")
    kind = "bf16" if wl.act == "bf16" else None
    lib.route(p, to_device(inp["x"], "cuda", kind), to_device(inp["w_router"], "cuda", kind),
              to_device(inp["bias"], "cuda"), ids, w, ws)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref["topk_ids"])
    np.testing.assert_allclose(w.cpu().numpy(), ref["topk_w"], rtol=W_RTOL, atol=0)


@pytest.mark.parametrize("T,E,k", [(1, 64, 8), (5, 200, 8), (16, 256, 8), (16, 33, 16), (40, 64, 8),
                                   (300, 200, 6)])
def test_route_with_exact_ties_matches_oracle(T, E, k):
    """Many equal logits: token rows are one-hot, so every logit is exactly one router weight
    (plus bias), and the router weights take five values (-1, -0, 0, 1, 2).  The selection must
    order them by value and then by expert index, like the oracle, on the single-launch path
    (moe_forward, up to 32 tokens) and on the one-wavefront-per-token path (moe_route)."""
    rng = np.random.default_rng(T * 7 + E)
    H, F = 256, 128
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), rng.integers(0, H, T)] = 1.0
    wr = rng.choice(np.array([-1.0, -0.0, 0.0, 1.0, 2.0], np.float32), size=(E, H))
    bias = rng.choice(np.array([0.0, 1.0], np.float32), size=E)
    wl = W("ties", T, H, E, k, F, "bf16", "bf16", 95, "none")
    inp = synth.generate(wl)
    inp.update(x=synth.to_bf16_bits(x), w_router=synth.to_bf16_bits(wr), bias=bias)
    ref = O.route(inp, k)
    note("route with ties T=%d E=%d k=%d" % (T, E, k))
    p = lib.problem(T, H, E, k, F)
    ws = torch.empty(lib.workspace_size(p), dtype=torch.uint8, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    xd, wd = to_device(inp["x"], "cuda", "bf16"), to_device(inp["w_router"], "cuda", "bf16")
    lib.route(p, xd, wd, to_device(bias, "cuda"), ids, w, ws)
    layer = MoELayer.from_workload(wl, inp)
    _, dbg = layer.forward(xd, debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref["topk_ids"])
    np.testing.assert_allclose(w.cpu().numpy(), ref["topk_w"], rtol=W_RTOL, atol=0)
    assert np.array_equal(dbg["topk_ids"].cpu().numpy(), ref["topk_ids"])
    for key in ("counts", "offsets", "sorted_token", "inv_perm"):
        assert np.array_equal(dbg[key].cpu().numpy().reshape(ref[key].shape), ref[key]), key


def test_route_small_and_large_batch_kernels_agree():
    """The router's wavefront shapes give the same logits: the screened router from 256 tokens
    (400), 4x4 (token, expert) blocks for 64 to 383, one token and two experts for 33 and 63
    tokens, one token and one expert while T * E <= 4096 (32, 17, 16 and 1 tokens at E = 128)."""
    wl = synth.WORKLOADS["decode64"].with_tokens(400, x_sub=400)
    inp = synth.generate(wl, with_experts=False)
    p400 = lib.problem(400, wl.hidden, wl.experts, wl.top_k, wl.ffn)
    ws = torch.empty(lib.workspace_size(p400), dtype=torch.uint8, device="cuda")
    x = to_device(inp["x"], "cuda", "bf16")
    wr = to_device(inp["w_router"], "cuda", "bf16")
    out = {}
    for T in (400, 383, 64, 63, 33, 32, 17, 16, 1):
        p = lib.problem(T, wl.hidden, wl.experts, wl.top_k, wl.ffn)
        ids = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
        note("route T=%d" % T)
        lib.route(p, x[:T], wr, None, ids, w, ws)
        out[T] = (ids.cpu().numpy(), w.cpu().numpy())
    for T in (383, 64, 63, 33, 32, 17, 16, 1):
        assert np.array_equal(out[400][0][:T], out[T][0]), T
        assert np.array_equal(out[400][1][:T], out[T][1]), T


# (T, H, E, k): the screen's K split is 4 for the 256-token cases and 1 at 8192 x 512; the token
# row sits in registers for H = 1024 and 2048, and goes through the generic form for H = 512
@pytest.mark.parametrize("T,H,E,k", [(256, 1024, 128, 8), (256, 1024, 256, 8), (256, 2048, 200, 6),
                                     (256, 512, 512, 16), (8192, 1024, 512, 8), (300, 1024, 16, 4)])
def test_screened_route_equals_full_router_on_hard_rows(T, H, E, k):
    """From 256 tokens, bf16 batches route through the screened router (approximate logits on
    the matrix cores, canonical logits only for the experts that can be selected); below 256 the
    full canonical router runs.  Routing T rows and their first 255 must give the same ids and
    weights bit for bit on those 255, on rows built to stress the screen: exact ties
    (duplicated router rows, zero tokens whose logits are the bias), near ties (router rows one
    bf16 step apart in one element), a token of norm 2^60 and non-finite tokens (both take the
    full row), bf16 subnormal tokens, and ordinary ones.  Ids of the finite rows must also equal
    the oracle's."""
    rng = np.random.default_rng(E * 31 + k + H)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    wr[1::7] = wr[0::7][: len(wr[1::7])]                       # exact duplicates
    wr[3::11] = wr[2::11][: len(wr[3::11])]
    bits = synth.to_bf16_bits(wr)
    bits[5::13, 17] = bits[4::13, 17][: len(bits[5::13, 17])] + 1  # one bf16 step apart
    bias = rng.choice(np.array([0.0, 0.25, 0.5], np.float32), size=E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[10:20] = 0.0                                              # logits = bias: ties everywhere
    x[20:30] *= 1e-39                                           # bf16 subnormals
    x[30] *= 2.0 ** 60                                          # norm above the screen's range
    x[31, 5] = np.inf
    x[32, 7] = np.nan
    x[33] = x[34]                                               # identical tokens
    xb = synth.to_bf16_bits(x)
    note("screened route T=%d H=%d E=%d k=%d" % (T, H, E, k))
    xd = to_device(xb, "cuda", "bf16")
    wd = to_device(bits, "cuda", "bf16")
    bd = to_device(bias, "cuda")
    out = {}
    for n in (T, 255):
        p = lib.problem(n, H, E, k, 128)
        ws = torch.empty(lib.workspace_size(p), dtype=torch.uint8, device="cuda")
        ids = torch.empty(n, k, dtype=torch.int32, device="cuda")
        w = torch.empty(n, k, dtype=torch.float32, device="cuda")
        lib.route(p, xd[:n], wd, bd, ids, w, ws)
        torch.cuda.synchronize()
        out[n] = (ids.cpu().numpy(), w.cpu().numpy())
    ids256, w256 = out[T]
    ids255, w255 = out[255]
    assert np.array_equal(ids256[:255], ids255)
    assert np.array_equal(w256[:255].view(np.uint32), w255.view(np.uint32))
    for r in range(T):  # every token: k distinct valid experts
        assert len(set(ids256[r].tolist())) == k and ids256[r].min() >= 0 and ids256[r].max() < E
    finite = np.isfinite(x).all(axis=1)
    ref = O.route({"x": xb[finite], "w_router": bits, "bias": bias}, k)
    assert np.array_equal(ids256[finite], ref["topk_ids"])
    keep = finite.copy()
    keep[30] = False  # its weights are a softmax of logits near 2^54: the oracle's fp64 differs
    np.testing.assert_allclose(w256[keep], ref["topk_w"][keep[finite]], rtol=W_RTOL, atol=0)


# ---------------------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (63, 128, 8), (64, 128, 8), (65, 256, 8),
                                   (1000, 128, 8), (300, 512, 16), (5, 4, 4), (4096, 128, 8)])
def test_permute_matches_oracle(T, E, k):
    rng = np.random.default_rng(T * 1000 + E + k)
    # skewed loads: draw experts with unequal probabilities, distinct within a token
    pr = rng.dirichlet(np.full(E, 0.3))
    ids = np.array([rng.choice(E, size=k, replace=False, p=pr) for _ in range(T)], dtype=np.int32)
    H = 256
    x = synth.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    note("permute T=%d E=%d k=%d" % (T, E, k))
    counts, offsets, st, ip = O.permute(ids, E)
    p = lib.problem(T, H, E, k, 128)
    ws = torch.empty(lib.workspace_size(p), dtype=torch.uint8, device="cuda")
    g = dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
             offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
             sorted_token=torch.empty(T * k, dtype=torch.int32, device="cuda"),
             inv_perm=torch.empty(T * k, dtype=torch.int32, device="cuda"))
    xd = to_device(x, "cuda", "bf16")
    x_perm = torch.empty(T * k, H, dtype=torch.bfloat16, device="cuda")
    lib.permute(p, dev_i32(ids), g["counts"], g["offsets"], g["sorted_token"], g["inv_perm"], ws,
                x=xd, x_perm=x_perm)
    torch.cuda.synchronize()
    assert np.array_equal(g["counts"].cpu().numpy(), counts)
    assert np.array_equal(g["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(g["sorted_token"].cpu().numpy(), st)
    assert np.array_equal(g["inv_perm"].cpu().numpy(), ip)
    assert np.array_equal(to_host(x_perm), x[st])


# ---------------------------------------------------------------------------------------
# grouped GEMMs
# ---------------------------------------------------------------------------------------

def _routed(wl, inp):
    r = O.route(inp, wl.top_k)
    expert_of_row = np.repeat(np.arange(wl.experts), r["counts"]).astype(np.int32)
    return r, expert_of_row


@pytest.mark.parametrize("name", ["tiny", "small_bf16", "small_bf16_rm", "small_nvfp4", "small_nvfp4_rm",
                                  "ragged_bf16", "ragged_bf16_rm", "ragged_nvfp4", "win4_nvfp4",
                                  "win4_nvfp4_rm", "ragged_f32"])
@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_gate_up_matches_oracle(name, path):
    wl, layout = case(name)
    inp = inputs_of(wl)
    note("gate_up %s path=%s" % (name, path))
    r, eor = _routed(wl, inp)
    ref = O.gate_up_rows(inp, wl.wdt, wl.ffn, r["sorted_token"], eor)
    layer = MoELayer.from_workload(wl, inp, path=path, weight_layout=layout)
    p = layer.problem_for(wl.tokens)
    ws = layer.workspace(wl.tokens)
    A = wl.assignments
    hid = layer.empty_act(A, wl.ffn)
    x = layer.act_tensor(inp["x"])
    lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x, dev_i32(r["sorted_token"]), dev_i32(r["offsets"]),
                     layer.weights, hid, ws)
    # the same rows handed over already permuted (a_rows = NULL)
    x_perm = x[torch.from_numpy(r["sorted_token"].astype(np.int64)).cuda()].contiguous()
    hid2 = layer.empty_act(A, wl.ffn)
    lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x_perm, None, dev_i32(r["offsets"]), layer.weights,
                     hid2, ws)
    torch.cuda.synchronize()
    got = act_f64(to_host(hid))
    e = rel_err(got, ref)
    note("  gate_up rel err %.3e" % e)
    assert e <= TOL
    assert torch.equal(hid, hid2)


@pytest.mark.parametrize("name", ["tiny", "small_bf16", "small_bf16_rm", "small_nvfp4", "small_nvfp4_rm",
                                  "ragged_bf16", "ragged_bf16_rm", "ragged_nvfp4", "win4_nvfp4",
                                  "win4_nvfp4_rm", "ragged_f32"])
@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_down_matches_oracle(name, path):
    wl, layout = case(name)
    inp = inputs_of(wl)
    note("down %s path=%s" % (name, path))
    r, eor = _routed(wl, inp)
    rng = np.random.default_rng(5)
    A = wl.assignments
    hid_host = rng.standard_normal((A, wl.ffn)).astype(np.float32) * 0.05
    if wl.act == "bf16":
        hid_host = synth.to_bf16_bits(hid_host)
    ref = O.down_rows(inp, wl.wdt, wl.hidden, act_f64(hid_host), eor)
    layer = MoELayer.from_workload(wl, inp, path=path, weight_layout=layout)
    p = layer.problem_for(wl.tokens)
    ws = layer.workspace(wl.tokens)
    y_perm = layer.empty_act(A, wl.hidden)
    lib.grouped_gemm(p, lib.DOWN, layer.act_tensor(hid_host), None, dev_i32(r["offsets"]),
                     layer.weights, y_perm, ws)
    torch.cuda.synchronize()
    e = rel_err(act_f64(to_host(y_perm)), ref)
    note("  down rel err %.3e" % e)
    assert e <= TOL


def _one_hot_down(wdt, layout, path, H, inp_edit=None, seed=21):
    """hid row r = unit vector at f_r through the down GEMM: y_perm[r, h] must be W2[e][h, f_r]
    exactly (every weight format decodes exactly to bf16), which pins the weight decode and the
    tile index maps.  Returns (GPU y_perm as float64, oracle)."""
    E, F = 3, 128
    wl = W("onehot", 1, H, E, 1, F, "bf16", wdt, seed, "none")
    inp = synth.generate(wl)
    inp.pop("w13_gscale", None)
    inp.pop("w2_gscale", None)  # per-expert scale 1.0: the product stays exact
    if inp_edit:
        inp_edit(inp)
    A = E * F
    f_of_row = np.tile(np.arange(F), E)
    e_of_row = np.repeat(np.arange(E), F).astype(np.int32)
    hid = np.zeros((A, F), np.float32)
    hid[np.arange(A), f_of_row] = 1.0
    hid_bits = synth.to_bf16_bits(hid)
    ref = O.down_rows(inp, wdt, H, act_f64(hid_bits), e_of_row)
    layer = MoELayer(A, H, E, 1, F, "bf16", wdt, inp, path=path, weight_layout=layout)
    want = lib.LAYOUT_PACKED if layout == "packed" and (wdt != "nvfp4" or H % 256 == 0) else lib.LAYOUT_ROW_MAJOR
    assert layer.layout == want
    p = layer.problem_for(A)
    ws = layer.workspace(A)
    y_perm = layer.empty_act(A, H)
    offsets = np.arange(E + 1, dtype=np.int32) * F
    lib.grouped_gemm(p, lib.DOWN, layer.act_tensor(hid_bits), None, dev_i32(offsets), layer.weights,
                     y_perm, ws)
    torch.cuda.synchronize()
    return act_f64(to_host(y_perm)), ref


@pytest.mark.parametrize("wdt,layout,H", [("bf16", "packed", 256), ("bf16", "row_major", 256),
                                          ("nvfp4", "row_major", 192), ("nvfp4", "packed", 256),
                                          ("nvfp4", "row_major", 256)])
@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_down_with_one_hot_rows_returns_exact_weights(wdt, layout, H, path):
    note("one-hot down wdt=%s layout=%s H=%d path=%s" % (wdt, layout, H, path))
    got, ref = _one_hot_down(wdt, layout, path, H)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("layout", ["row_major", "packed"])
@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_nvfp4_every_finite_e4m3_scale_decodes_exactly(layout, path):
    """Every finite non-negative E4M3 block scale, 0x00 to 0x7E, subnormals 0x01-0x07 (m 2^-9)
    included, written over the down weights' scales with per-expert scale 1: the one-hot rows
    must return e2m1 * e4m3 exactly ("CuTeDSL at Perplexity", section Blackwell support:
    16-element NVFP4 blocks; E4M3 per the OCP 8-bit formats).  Each code covers many blocks,
    and the nibbles hold every E2M1 code."""
    H = 256

    def sweep(inp):
        s2 = inp["w2_scale"]
        inp["w2_scale"] = (np.arange(s2.size) % 127).astype(np.uint8).reshape(s2.shape)
        q = inp["w2"]
        rng = np.random.default_rng(5)
        inp["w2"] = rng.integers(0, 256, q.shape).astype(np.uint8)

    note("NVFP4 scale sweep layout=%s path=%s" % (layout, path))
    got, ref = _one_hot_down("nvfp4", layout, path, H, inp_edit=sweep)
    assert np.all(np.isfinite(ref))
    sub = np.abs(ref)[(ref != 0)].min()
    assert sub <= 2.0 ** -9  # products of the subnormal scales are in the output
    assert np.array_equal(got, ref)


def test_packed_weight_layout_matches_its_definition():
    """The packed layout rebuilt independently with numpy from its definition in moe.h."""
    E, H, F = 2, 512, 256
    wl = W("pack", 1, H, E, 1, F, "bf16", "bf16", 71, "none")
    inp = synth.generate(wl)
    p = lib.problem(1, H, E, 1, F)
    w13 = to_device(inp["w13"], "cuda", "bf16")
    w2 = to_device(inp["w2"], "cuda", "bf16")
    p13, p2 = torch.empty_like(w13), torch.empty_like(w2)
    note("pack layout")
    lib.pack_weights(p, w13, w2, p13, p2)
    torch.cuda.synchronize()

    def expect(w, kind):
        K = H if kind == 0 else F
        tiles = F // 128 if kind == 0 else H // 256
        out = np.empty(w.size, dtype=np.uint16)
        i = 0
        for e in range(E):
            for t in range(tiles):
                for st in range(K // 32):
                    for r in range(256):
                        if kind == 0:
                            f = 128 * t + 64 * (r // 128) + (r % 64)
                            row = f if r % 128 < 64 else F + f
                        else:
                            row = 256 * t + r
                        for slot in range(4):
                            c = slot ^ ((r >> 1) & 3)
                            out[i:i + 8] = w[e, row, st * 32 + c * 8: st * 32 + c * 8 + 8]
                            i += 8
        return out

    assert np.array_equal(to_host(p13).ravel(), expect(inp["w13"], 0))
    assert np.array_equal(to_host(p2).ravel(), expect(inp["w2"], 1))


def test_packed_nvfp4_layout_matches_its_definition():
    """The packed NVFP4 bytes and scales rebuilt independently with numpy from their definition
    in moe.h (tiles of 256 rows in the bf16 row order; 16 bytes per row and stage, 4 scale bytes
    per row and stage pair)."""
    E, H, F = 2, 512, 256
    wl = W("pack4", 1, H, E, 1, F, "bf16", "nvfp4", 72, "none")
    inp = synth.generate(wl)
    p = lib.problem(1, H, E, 1, F, "bf16", "nvfp4")
    dev = {k: to_device(inp[k], "cuda") for k in ("w13", "w2", "w13_scale", "w2_scale")}
    out = {k: torch.empty_like(v) for k, v in dev.items()}
    note("packed NVFP4 layout")
    lib.pack_weights(p, dev["w13"], dev["w2"], out["w13"], out["w2"])
    lib.pack_scales(p, dev["w13_scale"], dev["w2_scale"], out["w13_scale"], out["w2_scale"])
    torch.cuda.synchronize()

    def expect(w, kind, unit):
        rows_of_tile, ntiles = 256, (F // 128 if kind == 0 else H // 256)
        out = []
        for e in range(E):
            for t in range(ntiles):
                for st in range(w.shape[2] // unit):
                    for r in range(rows_of_tile):
                        if kind == 0:
                            f = 128 * t + 64 * (r // 128) + (r % 64)
                            row = f if r % 128 < 64 else F + f
                        else:
                            row = 256 * t + r
                        out.append(w[e, row, st * unit:(st + 1) * unit])
        return np.concatenate(out)

    for key, kind, unit in (("w13", 0, 16), ("w2", 1, 16), ("w13_scale", 0, 4), ("w2_scale", 1, 4)):
        assert np.array_equal(out[key].cpu().numpy().ravel(), expect(inp[key], kind, unit)), key


@pytest.mark.parametrize("name", ["small_nvfp4", "win4_nvfp4", "small_bf16", "ragged_bf16",
                                  "small_mxfp8", "small_mxfp4", "split_mxfp8"])
def test_weight_layouts_agree(name):
    """Packed and row-major weights give the same layer: bit for bit on the bf16 and MX kernels
    and the NVFP4 prefill kernels (same values in the same LDS image or operand registers, other
    addresses), within the bar on the NVFP4 decode kernels (another order of K)."""
    wl = SMALL[name]
    inp = inputs_of(wl)
    a = MoELayer.from_workload(wl, inp, weight_layout="packed")
    b = MoELayer.from_workload(wl, inp, weight_layout="row_major")
    assert a.layout == lib.LAYOUT_PACKED and b.layout == lib.LAYOUT_ROW_MAJOR
    x = a.act_tensor(inp["x"])
    note("weight layouts %s" % name)
    ya = a.forward(x, path="prefill").clone()
    yb = b.forward(x, path="prefill").clone()
    da = a.forward(x, path="decode").clone()
    db = b.forward(x, path="decode")
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)
    if wl.wdt == "nvfp4":
        assert rel_err(act_f64(to_host(da)), act_f64(to_host(db))) <= TOL
    else:
        assert torch.equal(da, db)


def test_row_major_layer_matches_oracle():
    """A caller holding dense row-major bf16 weights gets the layer without packing them."""
    wl = SMALL["ragged_bf16"]
    inp = inputs_of(wl)
    note("row-major bf16 layer")
    layer = MoELayer.from_workload(wl, inp, weight_layout="row_major")
    assert layer.layout == lib.LAYOUT_ROW_MAJOR
    _check_forward(wl, inp, layer)


# ---------------------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_combine_matches_oracle(act):
    rng = np.random.default_rng(7)
    T, k, H = 300, 8, 256
    A = T * k
    ip = rng.permutation(A).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    yp = rng.standard_normal((A, H)).astype(np.float32)
    if act == "bf16":
        yp = synth.to_bf16_bits(yp)
    ref = O.combine(act_f64(yp), ip, w.astype(np.float64))
    p = lib.problem(T, H, 16, k, 128, act, act)
    y = torch.empty(T, H, dtype=torch.float32 if act == "f32" else torch.bfloat16, device="cuda")
    note("combine act=%s" % act)
    lib.combine(p, to_device(yp, "cuda"), dev_i32(ip), to_device(w, "cuda"), y)
    torch.cuda.synchronize()
    e = rel_err(act_f64(to_host(y)), ref)
    assert e <= (1e-6 if act == "f32" else 8e-3)


# ---------------------------------------------------------------------------------------
# the whole layer
# ---------------------------------------------------------------------------------------

def _check_forward(wl, inp, layer, tokens=None, path=None):
    x = layer.act_tensor(inp["x"])
    y, dbg = layer.forward(x, debug=True, path=path)
    torch.cuda.synchronize()
    ref = O.forward(inp, wl.top_k, wl.wdt, wl.ffn, wl.renormalize, tokens=tokens)
    for key in ("topk_ids", "counts", "offsets", "sorted_token", "inv_perm"):
        got = dbg[key].cpu().numpy()
        assert np.array_equal(got.reshape(ref[key].shape), ref[key]), key
    np.testing.assert_allclose(dbg["topk_w"].cpu().numpy(), ref["topk_w"], rtol=W_RTOL, atol=0)
    got = act_f64(to_host(y))[ref["tokens"]]
    e = rel_err(got, ref["y"])
    note("  %s y rel err %.3e, per-element p99 %.3e, over %d tokens"
         % (wl.name, e, p99_err(got, ref["y"]), len(ref["tokens"])))
    assert e <= TOL
    return y


FWD_CASES = ["tiny", "small_bf16", "small_nvfp4", "ragged_bf16", "ragged_nvfp4", "win4_nvfp4",
             "win4_nvfp4_rm", "ragged_f32", "decode1", "decode8", "nvfp4_decode", "nvfp4_decode_rm"]


@pytest.mark.parametrize("name", FWD_CASES)
def test_forward_matches_oracle(name):
    wl, layout = case(name)
    inp = inputs_of(wl)
    note("forward %s" % name)
    layer = MoELayer.from_workload(wl, inp, weight_layout=layout)
    _check_forward(wl, inp, layer)


def test_forward_decode64_every_token():
    """The 64-token decode batch: the whole layer output of every token against the oracle."""
    wl = synth.WORKLOADS["decode64"]
    inp = inputs_of(wl)
    note("forward decode64, all 64 tokens")
    _check_forward(wl, inp, MoELayer.from_workload(wl, inp))


@pytest.mark.parametrize("name", ["prefill", "nvfp4_prefill"])
def test_forward_full_size(name):
    """Full-size prefill layers: routing and dispatch of every token bit-exact, the layer output
    on a sample of tokens, and through the stage entry points every hid and y_perm row of the
    largest expert, a ragged one and the smallest one (gpu_checks)."""
    wl = synth.WORKLOADS[name]
    note("forward full size %s: generating inputs" % name)
    inp = inputs_of(wl)
    layer = MoELayer.from_workload(wl, inp)
    rng = np.random.default_rng(99)
    toks = np.unique(np.concatenate([[0, wl.tokens - 1], rng.choice(wl.tokens, 10, replace=False)]))
    note("forward full size %s: running" % name)
    _check_forward(wl, inp, layer, tokens=toks)
    note("forward full size %s: stage entry points, whole experts" % name)
    check_experts_through_stages(wl, inp, layer, note)
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["small_bf16", "small_nvfp4"])
def test_prefill_and_decode_paths_agree(name):
    wl = SMALL[name]
    inp = inputs_of(wl)
    layer = MoELayer.from_workload(wl, inp)
    x = layer.act_tensor(inp["x"])
    note("paths %s" % name)
    ya, da = layer.forward(x, debug=True, path="prefill")
    ya = ya.clone()
    yb, db = layer.forward(x, debug=True, path="decode")
    torch.cuda.synchronize()
    for key in ("topk_ids", "topk_w", "counts", "offsets", "sorted_token", "inv_perm"):
        assert torch.equal(da[key], db[key]), key
    assert rel_err(act_f64(to_host(ya)), act_f64(to_host(yb))) <= TOL


def test_forward_is_deterministic_and_scales_exactly():
    wl = SMALL["small_bf16"]
    inp = dict(inputs_of(wl))
    layer = MoELayer.from_workload(wl, inp)
    x = layer.act_tensor(inp["x"])
    note("determinism")
    y1 = layer.forward(x).clone()
    y2 = layer.forward(x).clone()
    assert torch.equal(y1, y2)
    # doubling the down weights (exact in bf16) doubles every output exactly
    inp2 = dict(inp)
    inp2["w2"] = synth.to_bf16_bits(bf16_bits_to_f64(inp["w2"]).astype(np.float32) * 2)
    layer2 = MoELayer.from_workload(wl, inp2)
    y3 = layer2.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y3.float(), (y1.float() * 2))


def test_token_permutation_permutes_outputs():
    wl = SMALL["small_bf16"]
    inp = inputs_of(wl)
    layer = MoELayer.from_workload(wl, inp)
    perm = np.random.default_rng(3).permutation(wl.tokens)
    note("token permutation")
    y = layer.forward(layer.act_tensor(inp["x"])).clone()
    yp = layer.forward(layer.act_tensor(inp["x"][perm]))
    torch.cuda.synchronize()
    assert torch.equal(yp, y[torch.from_numpy(perm).cuda()])


# ---------------------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------------------

def test_zero_tokens_is_a_no_op():
    wl = SMALL["small_bf16"]
    layer = MoELayer.from_workload(wl, inputs_of(wl))
    x = layer.empty_act(0, wl.hidden)
    y, dbg = layer.forward(x, debug=True)
    torch.cuda.synchronize()
    assert y.shape == (0, wl.hidden)
    assert int(dbg["counts"].abs().sum()) == 0 and int(dbg["offsets"].abs().sum()) == 0


@pytest.mark.parametrize("wdt", ["bf16", "nvfp4"])
def test_all_tokens_on_the_same_experts(wdt):
    wl = W("hot", 200, 256, 8, 2, 128, "bf16", wdt, 31, "normal")
    inp = synth.generate(wl)
    inp["bias"] = np.zeros(8, np.float32)
    inp["bias"][[6, 1]] = 1e4
    note("all tokens on experts 1, 6 wdt=%s" % wdt)
    layer = MoELayer.from_workload(wl, inp)
    _check_forward(wl, inp, layer)


@pytest.mark.parametrize("T,E,k", [(40, 4, 4), (40, 1, 1), (40, 16, 16), (300, 16, 16)])
def test_k_equals_e(T, E, k):
    """Every expert selected; at 300 tokens through the screened router, where every expert is a
    candidate."""
    wl = W("keqe", T, 256, E, k, 128, "bf16", "bf16", 41 + E, "normal")
    inp = synth.generate(wl)
    note("k=E=%d T=%d" % (E, T))
    _check_forward(wl, inp, MoELayer.from_workload(wl, inp))


@pytest.mark.parametrize("T,E,k", [(1, 8, 8), (8, 512, 16), (3, 5, 2), (8, 128, 8), (5, 1, 1),
                                   (2, 3, 3), (20, 64, 8), (32, 7, 3), (32, 512, 16)])
def test_small_batch_single_launch_dispatch(T, E, k):
    """Batches of up to 32 tokens select and dispatch in one single-block launch (up to four
    tokens per wavefront); routing outputs stay bit-exact and the layer output within tolerance."""
    wl = W("smallsel", T, 256, E, k, 128, "bf16", "bf16", 71 + E + T, "normal")
    inp = synth.generate(wl)
    note("small-batch dispatch T=%d E=%d k=%d" % (T, E, k))
    _check_forward(wl, inp, MoELayer.from_workload(wl, inp))


@pytest.mark.parametrize("T,E", [(50, 8), (300, 32)])
def test_full_softmax_weights_option(T, E):
    """Full-softmax weights (renormalize = 0) need every canonical logit, so batches the screened
    router would take (from 256 bf16 tokens) route through the full router instead."""
    wl = W("nr", T, 256, E, 3, 128, "bf16", "bf16", 51, "normal", renormalize=False)
    inp = synth.generate(wl)
    note("renormalize=0 T=%d E=%d" % (T, E))
    _check_forward(wl, inp, MoELayer.from_workload(wl, inp))


def test_single_token_prefill_path_and_large_batch_decode_path():
    for T, path in ((1, "prefill"), (600, "decode")):
        wl = W("force", T, 256, 32, 4, 128, "bf16", "nvfp4", 61, "normal")
        inp = synth.generate(wl)
        note("forced path %s T=%d" % (path, T))
        _check_forward(wl, inp, MoELayer.from_workload(wl, inp, path=path))


# ---------------------------------------------------------------------------------------
# limits, streams, non-finite inputs
# ---------------------------------------------------------------------------------------

def test_largest_expert_count_and_top_k_at_prefill_size():
    """E = 512 experts, k = 16 (the ABI's limits) with 2048 tokens: many partially filled
    tiles per launch on the prefill path; routing bit-exact, outputs on sampled tokens."""
    wl = W("maxek", 2048, 256, 512, 16, 128, "bf16", "bf16", 91, "normal")
    inp = synth.generate(wl)
    note("E=512 k=16 T=2048")
    layer = MoELayer.from_workload(wl, inp)
    toks = np.array([0, 1, 777, 1500, 2047])
    _check_forward(wl, inp, layer, tokens=toks)


def test_forward_on_a_side_stream_matches_the_default_stream():
    wl = SMALL["small_nvfp4"]
    inp = inputs_of(wl)
    layer = MoELayer.from_workload(wl, inp)
    x = layer.act_tensor(inp["x"])
    note("side stream")
    y0 = layer.forward(x).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y1 = layer.forward(x, stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(y0, y1)


def test_non_finite_inputs_stay_memory_safe_and_route_validly():
    """Non-finite activations give unspecified values but valid, distinct expert ids and a
    complete permutation (the header's promise)."""
    wl = W("nonfinite", 64, 256, 16, 4, 128, "bf16", "bf16", 93, "normal")
    inp = synth.generate(wl)
    x = inp["x"].copy()
    x[3, :] = 0x7FC0   # NaN
    x[5, 7] = 0x7F80   # +Inf
    x[9, 0] = 0xFF80   # -Inf
    inp["x"] = x
    layer = MoELayer.from_workload(wl, inp)
    note("non-finite inputs")
    for path in ("prefill", "decode"):
        y, dbg = layer.forward(layer.act_tensor(x), debug=True, path=path)
        torch.cuda.synchronize()
        ids = dbg["topk_ids"].cpu().numpy()
        assert ids.min() >= 0 and ids.max() < wl.experts
        assert all(len(set(r)) == wl.top_k for r in ids)
        ip = dbg["inv_perm"].cpu().numpy()
        assert np.array_equal(np.sort(ip), np.arange(wl.assignments))
        st = dbg["sorted_token"].cpu().numpy()
        assert np.array_equal(st[ip], np.arange(wl.assignments) // wl.top_k)
        good = [t for t in range(wl.tokens) if t not in (3, 5, 9)]
        assert np.isfinite(act_f64(to_host(y))[good]).all()


@pytest.mark.parametrize("name,T", [("decode1", 1), ("decode8", 8), ("nvfp4_decode", 3), ("small_bf16", 5),
                                    ("nvfp4_decode", 16), ("decode8", 32), ("decode8", 33), ("small_bf16", 384),
                                    ("ragged_bf16", 77), ("small_nvfp4", 384), ("k16_bf16", 1),
                                    ("small_bf16", 1), ("small_mxfp8", 5), ("small_mxfp8", 384),
                                    ("small_mxfp4", 5), ("small_mxfp4", 384), ("split_mxfp8", 4)])
def test_forward_equals_its_stages(name, T):
    """moe_forward must equal route -> permute -> two grouped GEMMs -> combine through the stage
    entry points, bit for bit: on batches of up to 32 tokens (single-block selection and
    dispatch; T = 33 is the first size past it), on the prefill kernels (the bf16 forward
    hands hid over in the packed tile image, the stage entry points row-major) and on the MX
    kernels (the forward's gate/up epilogue quantizes hid to MXFP8 itself, the stage entry
    points store bf16 hid and the down GEMM quantizes it)."""
    base = SMALL.get(name) or synth.WORKLOADS[name]
    wl = base.with_tokens(T, x_sub=100 + T)
    inp = inputs_of(wl)
    layer = MoELayer.from_workload(wl, inp)
    x = layer.act_tensor(inp["x"])
    note("forward vs stages %s T=%d" % (name, T))
    y_fused = layer.forward(x)
    p = layer.problem_for(T)
    ws = layer.workspace(T)
    A, dev = T * wl.top_k, "cuda"
    ids = torch.empty(T, wl.top_k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, wl.top_k, dtype=torch.float32, device=dev)
    counts = torch.empty(wl.experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(wl.experts + 1, dtype=torch.int32, device=dev)
    st = torch.empty(A, dtype=torch.int32, device=dev)
    ip = torch.empty(A, dtype=torch.int32, device=dev)
    lib.route(p, x, layer.w_router, layer.bias, ids, tw, ws)
    lib.permute(p, ids, counts, offsets, st, ip, ws)
    hid = layer.empty_act(A, wl.ffn)
    yp = layer.empty_act(A, wl.hidden)
    lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x, st, offsets, layer.weights, hid, ws)
    lib.grouped_gemm(p, lib.DOWN, hid, None, offsets, layer.weights, yp, ws)
    y_stages = layer.empty_act(T, wl.hidden)
    lib.combine(p, yp, ip, tw, y_stages)
    torch.cuda.synchronize()
    assert torch.equal(y_fused.view(torch.int16), y_stages.view(torch.int16))
