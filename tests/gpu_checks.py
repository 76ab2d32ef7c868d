"""Full-size parity through the stage entry points, shared by the GPU test modules.

At the full workload sizes the oracle cannot run every row, so these checks pick whole experts
whose row tiles exercise what a sampled token can miss: the most-loaded expert (many 256-row
tiles, the last one partial), an expert whose row count is not a multiple of 256 (a ragged last
tile), and the least-loaded expert (one row where the routing gives one, else the fewest).
Every row of those experts is compared element by element: hid from moe_grouped_gemm
(gate/up + SwiGLU) against the oracle's gate/up rows, and y_perm from moe_grouped_gemm (down)
against the oracle's down projection of the GPU's own hid (so the down GEMM is checked on its
own input).
"""
import numpy as np
import torch

from mixture_experts_layer_softmax_amd import lib
from mixture_experts_layer_softmax_amd.layer import bf16_bits_to_f64, to_host
from oracle import oracle as O

TOL = 2e-2


def pick_experts(counts):
    """(largest, ragged, smallest) expert ids: the most rows; the most rows among counts that are
    not a multiple of 256 (other than the largest); the fewest rows (at least one)."""
    counts = np.asarray(counts)
    order = np.argsort(-counts, kind="stable")
    big = int(order[0])
    ragged = next((int(e) for e in order if e != big and counts[e] % 256 and counts[e] > 256),
                  next(int(e) for e in order if e != big and counts[e] % 256))
    live = np.flatnonzero(counts > 0)
    small = int(live[np.argmin(counts[live])])
    return big, ragged, small


def p99_err(got, ref):
    """99th percentile over elements of |got - ref| / (|ref| + 1e-3 rms(ref)): the per-element
    figure reported beside the infinity-norm relative error (the floor keeps elements near zero
    from dominating)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    d = np.abs(got - ref) / (np.abs(ref) + 1e-3 * rms + 1e-300)
    return float(np.percentile(d, 99)) if d.size else 0.0


def block_err(got, ref):
    """max |got - ref| / max |ref| over a block of rows."""
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def check_experts_through_stages(wl, inp, layer, note):
    """Route and dispatch on the GPU (checked bit-exact against the oracle), run both grouped
    GEMMs through the stage entry points over all rows, and compare every row of three experts
    (pick_experts) with the oracle."""
    x = layer.act_tensor(inp["x"])
    p = layer.problem_for(wl.tokens)
    ws = layer.workspace(wl.tokens)
    A, dev = wl.assignments, layer.device
    ids = torch.empty(wl.tokens, wl.top_k, dtype=torch.int32, device=dev)
    tw = torch.empty(wl.tokens, wl.top_k, dtype=torch.float32, device=dev)
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
    torch.cuda.synchronize()
    ref = O.route(inp, wl.top_k, wl.renormalize)
    for key, t in (("topk_ids", ids), ("counts", counts), ("offsets", offsets), ("sorted_token", st),
                   ("inv_perm", ip)):
        assert np.array_equal(t.cpu().numpy().reshape(ref[key].shape), ref[key]), key
    off = ref["offsets"]
    hid_h = to_host(hid)
    yp_h = to_host(yp)
    for e in pick_experts(ref["counts"]):
        r0, r1 = int(off[e]), int(off[e + 1])
        note("  %s expert %d: rows %d..%d (%d rows, %d full 256-row tiles)"
             % (wl.name, e, r0, r1, r1 - r0, (r1 - r0) // 256))
        rows_e = np.full(r1 - r0, e, np.int32)
        ref_hid = O.gate_up_rows(inp, wl.wdt, wl.ffn, ref["sorted_token"][r0:r1], rows_e)
        got_hid = bf16_bits_to_f64(hid_h[r0:r1])
        eh = block_err(got_hid, ref_hid)
        ref_y = O.down_rows(inp, wl.wdt, wl.hidden, got_hid, rows_e)
        ey = block_err(bf16_bits_to_f64(yp_h[r0:r1]), ref_y)
        note("    hid rel err %.3e, y_perm rel err %.3e" % (eh, ey))
        assert eh <= TOL and ey <= TOL, (e, eh, ey)
