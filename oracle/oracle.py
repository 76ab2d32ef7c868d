"""Python face of the CPU oracle in ``moe_oracle.c``.

TEST INFRASTRUCTURE ONLY: only the test-suite, the smoke check and the benchmark's CPU
baseline may import this module.  It never touches the GPU library and shares no code with
it; inputs come from the seeded generator as plain numpy arrays.

The steps and the readings they take are documented in ``moe_oracle.c``; this file only
marshals arrays (argument checking and dtype plumbing, no arithmetic of the layer).
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_OUT = os.path.join(_HERE, "_build", "libmoe_oracle.so")

F32, BF16, NVFP4, MXFP8, MXFP4 = 0, 1, 2, 3, 4
_DT = {"f32": F32, "bf16": BF16, "nvfp4": NVFP4, "mxfp8": MXFP8, "mxfp4": MXFP4}

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FP contraction, OpenMP)."""
    if force or not os.path.exists(_OUT) or os.path.getmtime(_OUT) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(_OUT), exist_ok=True)
        tmp = _OUT + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _OUT)
    return _OUT


def _P(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def lib() -> C.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            path = _OUT if os.path.exists(_OUT) else build()
            L = C.CDLL(path)
            i64, i32, vp = C.c_int64, C.c_int, C.c_void_p
            L.oracle_logit.restype = C.c_float
            L.oracle_logit.argtypes = [vp, vp, i32, i64, i32, C.c_float]
            L.oracle_router_logits.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp]
            L.oracle_select.argtypes = [i64, i64, i32, vp, i32, vp, vp]
            L.oracle_permute.argtypes = [i64, i32, i64, i64, i64, vp, vp, vp, vp, vp]
            L.oracle_expert_rows.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64,
                                             vp, vp, vp, vp]
            L.oracle_down_rows.argtypes = [i64, i64, i32, vp, vp, vp, i64, vp, vp, vp]
            L.oracle_combine.argtypes = [i64, i32, i64, vp, vp, vp, vp]
            for n in ("oracle_decode_bf16", "oracle_decode_e2m1", "oracle_decode_e4m3", "oracle_decode_e8m0"):
                getattr(L, n).argtypes = [vp, vp, i64]
            L.oracle_mx_quantize.argtypes = [vp, i64, vp, vp, vp]
            L.oracle_set_threads.argtypes = [i32]
            L.oracle_max_threads.restype = i32
            _lib = L
    return _lib


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


# ---------------------------------------------------------------------------------------
# codecs (exposed for the codec pins)
# ---------------------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_decode_bf16(_P(b), _P(out), b.size)
    return out


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().oracle_decode_e2m1(_P(c), _P(out), c.size)
    return out


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().oracle_decode_e4m3(_P(c), _P(out), c.size)
    return out


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().oracle_decode_e8m0(_P(c), _P(out), c.size)
    return out


def mx_quantize(values: np.ndarray):
    """MX (E4M3 + E8M0 per 32 along the last axis) quantization of values given as float64,
    float32 or bf16 bits: returns (codes uint8 [..., K], scales uint8 [..., K/32],
    decoded float64 [..., K])."""
    v = values
    if v.dtype == np.uint16:
        v = decode_bf16(v)
    v = np.ascontiguousarray(v, dtype=np.float64)
    assert v.shape[-1] % 32 == 0
    codes = np.empty(v.shape, dtype=np.uint8)
    scales = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), dtype=np.uint8)
    dec = np.empty(v.shape, dtype=np.float64)
    lib().oracle_mx_quantize(_P(v), v.size // 32, _P(codes), _P(scales), _P(dec))
    return codes, scales, dec


# ---------------------------------------------------------------------------------------
# the layer's steps
# ---------------------------------------------------------------------------------------

def _act_dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("activations must be float32 or bf16 bits (uint16), got %s" % a.dtype)


def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    x = np.ascontiguousarray(x)
    w_router = np.ascontiguousarray(w_router)
    dt = _act_dt(x)
    assert w_router.dtype == x.dtype and x.shape[1] == w_router.shape[1] and x.shape[1] % 8 == 0
    T, H = x.shape
    E = w_router.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, E), dtype=np.float32)
    lib().oracle_router_logits(T, H, E, dt, _P(x), _P(w_router), _P(b), _P(out))
    return out


def select(logits: np.ndarray, k: int, renormalize: bool = True):
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    assert 1 <= k <= E
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_select(T, E, int(k), _P(lg), int(bool(renormalize)), _P(ids), _P(w))
    return ids, w


def _held(num_experts: int, held):
    if held is None:
        return 0, num_experts
    b, n = int(held[0]), int(held[1])
    assert 0 <= b and 0 < n and b + n <= num_experts
    return b, b + n


def permute(ids: np.ndarray, num_experts: int, held=None):
    """Dispatch; ``held = (begin, count)`` keeps only the assignments of experts
    [begin, begin + count) (expert parallelism), the others get inv_perm = -1.
    ``sorted_token`` has offsets[E] meaningful entries."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    A = T * k
    eb, ee = _held(num_experts, held)
    counts = np.empty(num_experts, dtype=np.int32)
    offsets = np.empty(num_experts + 1, dtype=np.int32)
    sorted_token = np.full(A, -1, dtype=np.int32)
    inv_perm = np.empty(A, dtype=np.int32)
    lib().oracle_permute(T, int(k), num_experts, eb, ee, _P(ids), _P(counts), _P(offsets),
                         _P(sorted_token), _P(inv_perm))
    return counts, offsets, sorted_token, inv_perm


def expert_rows(inputs: dict, wdt: str, ffn: int, row_token, row_expert, want_hid=False):
    """Expert FFN of the given (token, expert) rows in double: returns out[n, H] (, hid[n, F])."""
    x = np.ascontiguousarray(inputs["x"])
    T, H = x.shape
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    re = np.ascontiguousarray(row_expert, dtype=np.int32)
    n = rt.size
    out = np.empty((n, H), dtype=np.float64)
    hid = np.empty((n, ffn), dtype=np.float64) if want_hid else None
    g = lambda k: None if inputs.get(k) is None else np.ascontiguousarray(inputs[k])
    w13, w2 = g("w13"), g("w2")
    s13, s2, g13, g2 = g("w13_scale"), g("w2_scale"), g("w13_gscale"), g("w2_gscale")
    if wdt in ("nvfp4", "mxfp8", "mxfp4"):
        assert w13.dtype == np.uint8 and s13 is not None and s2 is not None
    lib().oracle_expert_rows(H, ffn, _act_dt(x), _DT[wdt], _P(x), _P(w13), _P(w2), _P(s13), _P(s2),
                             _P(g13), _P(g2), n, _P(rt), _P(re), _P(out), _P(hid))
    return (out, hid) if want_hid else out


def gate_up_rows(inputs: dict, wdt: str, ffn: int, row_token, row_expert):
    """hid[n, F] = silu(gate) * up of the given (token, expert) rows, in double."""
    x = np.ascontiguousarray(inputs["x"])
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    re = np.ascontiguousarray(row_expert, dtype=np.int32)
    hid = np.empty((rt.size, ffn), dtype=np.float64)
    g = lambda k: None if inputs.get(k) is None else np.ascontiguousarray(inputs[k])
    lib().oracle_expert_rows(x.shape[1], ffn, _act_dt(x), _DT[wdt], _P(x), _P(g("w13")), _P(g("w2")),
                             _P(g("w13_scale")), _P(g("w2_scale")), _P(g("w13_gscale")),
                             _P(g("w2_gscale")), rt.size, _P(rt), _P(re), None, _P(hid))
    return hid


def down_rows(inputs: dict, wdt: str, hidden: int, hid: np.ndarray, row_expert):
    """out[n, H] = W2[e] . hid[n] for the given rows (hid given as double)."""
    h = np.ascontiguousarray(hid, dtype=np.float64)
    re = np.ascontiguousarray(row_expert, dtype=np.int32)
    out = np.empty((re.size, hidden), dtype=np.float64)
    g = lambda k: None if inputs.get(k) is None else np.ascontiguousarray(inputs[k])
    lib().oracle_down_rows(hidden, h.shape[1], _DT[wdt], _P(g("w2")), _P(g("w2_scale")),
                           _P(g("w2_gscale")), re.size, _P(re), _P(h), _P(out))
    return out


def combine(y_perm: np.ndarray, inv_perm: np.ndarray, w: np.ndarray) -> np.ndarray:
    yp = np.ascontiguousarray(y_perm, dtype=np.float64)
    ip = np.ascontiguousarray(inv_perm, dtype=np.int32).ravel()
    ww = np.ascontiguousarray(w, dtype=np.float64)
    T, k = ww.shape
    H = yp.shape[1]
    y = np.empty((T, H), dtype=np.float64)
    lib().oracle_combine(T, int(k), H, _P(yp), _P(ip), _P(ww), _P(y))
    return y


def route(inputs: dict, top_k: int, renormalize: bool = True, held=None) -> dict:
    """Router logits, selection, weights and the dispatch permutation of every token
    (``held``: see permute)."""
    logits = router_logits(inputs["x"], inputs["w_router"], inputs.get("bias"))
    E = logits.shape[1]
    ids, w = select(logits, top_k, renormalize)
    counts, offsets, sorted_token, inv_perm = permute(ids, E, held)
    return dict(logits=logits, topk_ids=ids, topk_w=w, counts=counts, offsets=offsets,
                sorted_token=sorted_token, inv_perm=inv_perm)


def forward(inputs: dict, top_k: int, wdt: str, ffn: int, renormalize: bool = True,
            tokens=None, routed: dict | None = None, held=None) -> dict:
    """The whole layer.  ``tokens`` (optional) restricts the expert FFN and combine to a
    sample of tokens; routing and dispatch always cover every token.  ``y`` then has one row
    per sampled token, in the order given.  ``held = (begin, count)``: expert parallelism, the
    inputs hold the weights of experts [begin, begin + count) only and ``y`` is this share's
    partial output (see permute)."""
    r = routed if routed is not None else route(inputs, top_k, renormalize, held)
    T = r["topk_ids"].shape[0]
    eb = 0 if held is None else int(held[0])
    toks = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    k = top_k
    # rows of the permuted buffer that the chosen tokens own, found through inv_perm
    slots = (toks[:, None] * k + np.arange(k)[None, :]).ravel()
    pos_all = r["inv_perm"][slots]
    kept = pos_all >= 0
    pos = pos_all[kept]
    expert_of_pos = np.searchsorted(r["offsets"], pos, side="right") - 1
    rows = expert_rows(inputs, wdt, ffn, r["sorted_token"][pos], expert_of_pos - eb)
    # combine through a compact y_perm holding just those rows (-1: not dispatched here)
    local = np.full(pos_all.size, -1, dtype=np.int32)
    local[kept] = np.arange(pos.size, dtype=np.int32)
    y = combine(rows, local.reshape(toks.size, k), r["topk_w"][toks])
    out = dict(r)
    out.update(y=y, tokens=toks)
    return out
