"""GPU parity of one expert-parallel rank's share of the layer (held expert range).

With replicated inputs every rank routes all tokens, dispatches only the assignments of the
experts it holds and combines them into a partial output; the partial outputs of a partition
of the experts sum to the layer ("CuTeDSL at Perplexity", section Mixture-of-Experts
Dispatch/Combine; "Hosting Qwen on Blackwell", section Expert Parallel).  Bar as in
test_gpu_parity: routing and dispatch bit-exact (dispatch rows up to offsets[E]; inv_perm
including its -1 entries), outputs within 2e-2 of the oracle's partial output.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_softmax_amd import lib, synth
from mixture_experts_layer_softmax_amd.layer import MoELayer, bf16_bits_to_f64, to_device, to_host
from gpu_checks import p99_err
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2
W_RTOL = 1e-5
W = synth.Workload

CASES = {
    "small_bf16": W("small_bf16", 512, 512, 8, 2, 256, "bf16", "bf16", 11, "normal"),
    "small_nvfp4": W("small_nvfp4", 384, 512, 16, 4, 256, "bf16", "nvfp4", 12, "normal"),
    "ragged_f32": W("ragged_f32", 33, 128, 5, 2, 192, "f32", "f32", 16, "normal"),
    "decode1": synth.WORKLOADS["decode1"],
    "decode8": synth.WORKLOADS["decode8"],
    "decode64": synth.WORKLOADS["decode64"],
}


def note(msg):
    print("[gpu] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _env():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib.load()
    O.build()


def act_f64(a):
    return a.astype(np.float64) if a.dtype == np.float32 else bf16_bits_to_f64(a)


def rel_err(y, ref):
    return float(np.max(np.abs(y - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def share(inp, b, n):
    out = dict(inp)
    for key in ("w13", "w2", "w13_scale", "w2_scale", "w13_gscale", "w2_gscale"):
        if inp.get(key) is not None:
            out[key] = np.ascontiguousarray(inp[key][b:b + n])
    return out


def run_share(wl, sub, b, n, tokens=None, path=None):
    """Forward of the share holding experts [b, b+n) on the GPU (``sub``: every token, the held
    experts' weights), checked against the oracle."""
    layer = MoELayer.from_workload(wl, sub, expert_begin=b, local_experts=n)
    x = layer.act_tensor(sub["x"])
    y, dbg = layer.forward(x, debug=True, path=path)
    torch.cuda.synchronize()
    ref = O.forward(sub, wl.top_k, wl.wdt, wl.ffn, wl.renormalize, tokens=tokens, held=(b, n))
    for key in ("topk_ids", "counts", "offsets", "inv_perm"):
        got = dbg[key].cpu().numpy()
        assert np.array_equal(got.reshape(ref[key].shape), ref[key]), key
    a_local = int(ref["offsets"][-1])
    assert np.array_equal(dbg["sorted_token"].cpu().numpy()[:a_local], ref["sorted_token"][:a_local])
    np.testing.assert_allclose(dbg["topk_w"].cpu().numpy(), ref["topk_w"], rtol=W_RTOL, atol=0)
    got = act_f64(to_host(y))[ref["tokens"]]
    e = rel_err(got, ref["y"])
    note("  %s experts [%d, %d): %d of %d rows, y rel err %.3e, per-element p99 %.3e"
         % (wl.name, b, b + n, a_local, wl.assignments, e, p99_err(got, ref["y"])))
    assert e <= TOL
    return got, ref


@pytest.mark.parametrize("name,b,n", [("small_bf16", 0, 3), ("small_bf16", 3, 5), ("small_bf16", 7, 1),
                                      ("small_nvfp4", 4, 8), ("ragged_f32", 1, 3), ("decode1", 0, 64),
                                      ("decode1", 64, 64), ("decode8", 32, 32),
                                      ("decode64", 96, 32)])
def test_share_matches_oracle(name, b, n):
    wl = CASES[name]
    note("expert-parallel share %s [%d, %d)" % (name, b, b + n))
    run_share(wl, synth.generate(wl, experts=range(b, b + n)), b, n)


@pytest.mark.parametrize("name,parts", [("small_bf16", ((0, 2), (2, 3), (5, 3))),
                                        ("small_nvfp4", ((0, 4), (4, 4), (8, 4), (12, 4)))])
def test_partial_outputs_of_a_partition_sum_to_the_layer(name, parts):
    wl = CASES[name]
    inp = synth.generate(wl)
    note("partition %s" % name)
    total = 0.0
    for b, n in parts:
        got, _ = run_share(wl, share(inp, b, n), b, n)
        total = total + got
    ref = O.forward(inp, wl.top_k, wl.wdt, wl.ffn, wl.renormalize)
    e = rel_err(total, ref["y"])
    note("  sum of %d partial outputs vs the layer: rel err %.3e" % (len(parts), e))
    assert e <= TOL


def test_permute_of_a_held_range_matches_oracle():
    rng = np.random.default_rng(31)
    T, E, k, b, n = 700, 64, 6, 16, 24
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, st, ip = O.permute(ids, E, held=(b, n))
    p = lib.problem(T, 256, E, k, 128, "bf16", "bf16", expert_begin=b, local_experts=n)
    ws = torch.empty(lib.workspace_size(p), dtype=torch.uint8, device="cuda")
    g = [torch.full((m,), -7, dtype=torch.int32, device="cuda") for m in (E, E + 1, T * k, T * k)]
    note("moe_permute held [%d, %d)" % (b, b + n))
    lib.permute(p, torch.from_numpy(ids).cuda(), *g, ws)
    torch.cuda.synchronize()
    assert np.array_equal(g[0].cpu().numpy(), counts)
    assert np.array_equal(g[1].cpu().numpy(), offsets)
    a_local = int(offsets[-1])
    assert np.array_equal(g[2].cpu().numpy()[:a_local], st[:a_local])
    assert np.array_equal(g[3].cpu().numpy(), ip)


@pytest.mark.parametrize("kind", [lib.GATE_UP_SWIGLU, lib.DOWN])
def test_grouped_gemm_leaves_rows_of_experts_not_held_untouched(kind):
    """Standalone grouped GEMM with a held range: rows of held experts match the oracle, rows
    that the offsets give to other experts are never written."""
    wl = W("gg", 64, 256, 8, 2, 128, "bf16", "bf16", 21, "none")
    b, n = 2, 4
    full = synth.generate(wl)
    sub = share(full, b, n)
    layer = MoELayer.from_workload(wl, sub, expert_begin=b, local_experts=n)
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 30, size=wl.experts).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(offsets[-1])
    p = lib.problem(A, wl.hidden, wl.experts, 1, wl.ffn, "bf16", "bf16", path="prefill",
                    expert_begin=b, local_experts=n)
    ws = torch.empty(lib.workspace_size(p), dtype=torch.uint8, device="cuda")
    expert_of_row = np.repeat(np.arange(wl.experts), counts)
    held = (expert_of_row >= b) & (expert_of_row < b + n)
    if kind == lib.GATE_UP_SWIGLU:
        a_host = synth.to_bf16_bits(rng.standard_normal((A, wl.hidden)).astype(np.float32))
        out = torch.full((A, wl.ffn), 7.0, dtype=torch.bfloat16, device="cuda")
        ref = O.gate_up_rows(dict(sub, x=a_host), "bf16", wl.ffn, np.arange(A)[held],
                             expert_of_row[held] - b)
    else:
        a_host = synth.to_bf16_bits(rng.standard_normal((A, wl.ffn)).astype(np.float32) * 0.1)
        out = torch.full((A, wl.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
        ref = O.down_rows(sub, "bf16", wl.hidden, bf16_bits_to_f64(a_host)[held], expert_of_row[held] - b)
    note("grouped gemm kind %d held [%d, %d)" % (kind, b, b + n))
    lib.grouped_gemm(p, kind, to_device(a_host, "cuda"), None, torch.from_numpy(offsets).cuda(),
                     layer.weights, out, ws)
    torch.cuda.synchronize()
    got = act_f64(to_host(out))
    assert np.all(got[~held] == 7.0)
    e = rel_err(got[held], ref)
    note("  held rows rel err %.3e" % e)
    assert e <= TOL


def test_prefill6000_share_of_four_ranks_sampled():
    """The pages' ~6000-token prefill (about 375 rows per expert) as the share of one of four
    expert-parallel ranks (32 of 128 experts), at full size, outputs on sampled tokens."""
    wl = synth.WORKLOADS["prefill6000"]
    b, n = 32, 32
    note("prefill6000 share [%d, %d): generating inputs" % (b, b + n))
    inp = synth.generate(wl, experts=range(b, b + n))  # every token, the held experts' weights
    layer = MoELayer.from_workload(wl, inp, expert_begin=b, local_experts=n)
    x = layer.act_tensor(inp["x"])
    y, dbg = layer.forward(x, debug=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    toks = np.unique(np.concatenate([[0, wl.tokens - 1], rng.choice(wl.tokens, 10, replace=False)]))
    note("prefill6000 share: oracle")
    ref = O.forward(inp, wl.top_k, wl.wdt, wl.ffn, tokens=toks, held=(b, n))
    for key in ("topk_ids", "counts", "offsets", "inv_perm"):
        assert np.array_equal(dbg[key].cpu().numpy().reshape(ref[key].shape), ref[key]), key
    a_local = int(ref["offsets"][-1])
    assert np.array_equal(dbg["sorted_token"].cpu().numpy()[:a_local], ref["sorted_token"][:a_local])
    got = act_f64(to_host(y))[toks]
    e = rel_err(got, ref["y"])
    note("  %d of %d rows held; y rel err %.3e, per-element p99 %.3e, on %d tokens"
         % (a_local, wl.assignments, e, p99_err(got, ref["y"]), toks.size))
    assert e <= TOL


@pytest.mark.parametrize("ep", [1, 8])
def test_grouped_gemm_one_token_per_expert_full_size(ep):
    """The grouped MoE GEMM benchmark shape of "Hosting Qwen on Blackwell" (every expert given
    one token; hidden 4096, expert ffn 1536), for all 128 experts and for one rank of eight:
    the gate/up + SwiGLU and down launches against the oracle's expert rows."""
    E, H, F = 128, 4096, 1536
    n = E // ep
    b = (ep - 1) * n
    wl = W("grouped1", n, H, E, 1, F, "bf16", "bf16", 707, "none")
    note("grouped gemm, one token for each of experts [%d, %d)" % (b, b + n))
    inp = synth.generate(wl, experts=range(b, b + n))
    held = dict(expert_begin=b, local_experts=n) if n < E else {}
    layer = MoELayer.from_workload(wl, inp, **held)
    p = layer.problem_for(n)
    ws = layer.workspace(n)
    x = layer.act_tensor(inp["x"])
    offsets = torch.from_numpy(np.clip(np.arange(E + 1) - b, 0, n).astype(np.int32)).cuda()
    hid = layer.empty_act(n, F)
    yp = layer.empty_act(n, H)
    lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, x, None, offsets, layer.weights, hid, ws)
    lib.grouped_gemm(p, lib.DOWN, hid, None, offsets, layer.weights, yp, ws)
    torch.cuda.synchronize()
    ref_y, ref_h = O.expert_rows(inp, "bf16", F, np.arange(n), np.arange(n), want_hid=True)
    eh = rel_err(act_f64(to_host(hid)), ref_h)
    ey = rel_err(act_f64(to_host(yp)), ref_y)
    note("  hid rel err %.3e, y rel err %.3e" % (eh, ey))
    assert eh <= TOL and ey <= TOL


@pytest.mark.parametrize("wdt", ["bf16", "nvfp4"])
def test_grouped_gemm_with_no_held_rows_after_one_with_rows(wdt):
    """Two standalone gate/up GEMMs in one workspace, of the same size: the first gives the held
    experts rows, the second gives every row to experts not held.  The prefill kernels split the
    tile list over the XCDs by ranges kept in the workspace; the second call's empty list must
    empty every range, so it writes no row (the first call's ranges would name its stale tiles)."""
    wl = W("gg0", 64, 512, 8, 2, 256, "bf16", wdt, 22, "none")
    b, n = 2, 3
    sub = share(synth.generate(wl), b, n)
    layer = MoELayer.from_workload(wl, sub, expert_begin=b, local_experts=n)
    A = 600
    p = lib.problem(A, wl.hidden, wl.experts, 1, wl.ffn, "bf16", wdt, path="prefill",
                    expert_begin=b, local_experts=n)
    ws = torch.empty(lib.workspace_size(p), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(8)
    a_host = synth.to_bf16_bits(rng.standard_normal((A, wl.hidden)).astype(np.float32))
    a = to_device(a_host, "cuda")
    first = np.array([10, 20, 300, 40, 200, 10, 10, 10], dtype=np.int32)  # held: 300, 40, 200
    second = np.array([100, 100, 0, 0, 0, 200, 100, 100], dtype=np.int32)
    for i, counts in enumerate((first, second)):
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        assert int(offsets[-1]) == A
        expert_of_row = np.repeat(np.arange(wl.experts), counts)
        held = (expert_of_row >= b) & (expert_of_row < b + n)
        out = torch.full((A, wl.ffn), 7.0, dtype=torch.bfloat16, device="cuda")
        note("grouped gemm %s call %d: %d held rows" % (wdt, i + 1, int(held.sum())))
        lib.grouped_gemm(p, lib.GATE_UP_SWIGLU, a, None, torch.from_numpy(offsets).cuda(),
                         layer.weights, out, ws)
        torch.cuda.synchronize()
        got = act_f64(to_host(out))
        assert np.all(got[~held] == 7.0)
        if held.any():
            ref = O.gate_up_rows(dict(sub, x=a_host), wdt, wl.ffn, np.arange(A)[held],
                                 expert_of_row[held] - b)
            e = rel_err(got[held], ref)
            note("  held rows rel err %.3e" % e)
            assert e <= TOL
