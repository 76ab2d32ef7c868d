"""The C-ABI library on the host (no GPU): it loads, exports every symbol ``include/moe.h``
declares, and rejects bad arguments before touching the device."""
import ctypes as C
import os
import re

import pytest

from mixture_experts_layer_softmax_amd import lib, synth

INCLUDE = os.path.join(os.path.dirname(__file__), "..", "include")


def declared():
    text = "".join(open(os.path.join(INCLUDE, f)).read() for f in sorted(os.listdir(INCLUDE))
                   if f.endswith(".h"))
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        from mixture_experts_layer_softmax_amd import build

        build.build()
    return lib.load()


def test_every_declared_symbol_is_exported(L):
    names = declared()
    assert set(names) == set(lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert lib.status_string(lib.MOE_OK) == "ok"
    assert "workspace" in lib.status_string(lib.MOE_ERR_WORKSPACE_TOO_SMALL)
    assert "static scratch" in lib.status_string(lib.MOE_ERR_SCRATCH_TOO_SMALL)
    assert lib.status_string(99) == "unknown status"


def test_forward_static_validation(L):
    """moe_forward_static validates the problem and refuses one that does not fit its static
    scratch before any HIP call (so these run without a GPU)."""
    V = C.c_void_p
    w = lib.ExpertWeights(FAKE, FAKE, None, None, None, None, 1)
    bad = lib.problem(16, 256, 8, 0, 128)  # k = 0
    assert L.moe_forward_static(C.byref(bad), V(FAKE), V(FAKE), None, C.byref(w), V(FAKE), None, None,
                                None, None, None, None, None) == lib.MOE_ERR_INVALID_ARGUMENT
    big = lib.problem(4096, 4096, 128, 8, 1536)
    assert lib.workspace_size(big) > lib.STATIC_SCRATCH_BYTES
    assert L.moe_forward_static(C.byref(big), V(FAKE), V(FAKE), None, C.byref(w), V(FAKE), None, None,
                                None, None, None, None, None) == lib.MOE_ERR_SCRATCH_TOO_SMALL
    # the decode shapes fit: 64 tokens of the 4096 x 1536 layer, 16 of the 256-expert NVFP4 one
    assert lib.workspace_size(lib.problem(64, 4096, 128, 8, 1536)) <= lib.STATIC_SCRATCH_BYTES
    assert lib.workspace_size(lib.problem(16, 4096, 256, 8, 2048, wdt="nvfp4")) <= lib.STATIC_SCRATCH_BYTES


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_workspace_size_of_every_workload(L, name):
    wl = synth.WORKLOADS[name]
    p = lib.problem(wl.tokens, wl.hidden, wl.experts, wl.top_k, wl.ffn, wl.act, wl.wdt)
    n = lib.workspace_size(p)
    A = wl.assignments
    # the intermediates dominate: hid [A,F] and y_perm [A,H] (+ their MXFP8 copies: codes and
    # scales); the bf16 prefill forward keeps hid as full 256-row tiles (the worst-case tile
    # count: ceil(A / 256) + min(A, E) + 1)
    act = 4 if wl.act == "f32" else 2
    hid_rows = A
    if wl.wdt == "bf16" and A >= 16 * wl.experts:
        hid_rows = ((A + 255) // 256 + min(A, wl.experts) + 1) * 256
    inter = (hid_rows * wl.ffn + A * wl.hidden) * act
    if wl.wdt.startswith("mx"):
        inter += A * (wl.ffn + wl.hidden) * 33 // 32
    assert n >= inter
    assert n < inter + 64 * 2 ** 20


FAKE = 1 << 20  # an aligned address that is never dereferenced: validation fails first


def _call_route(L, p, x=FAKE, wr=FAKE, ids=FAKE, w=FAKE, ws=FAKE, nbytes=1 << 40):
    V = C.c_void_p
    return L.moe_route(C.byref(p), V(x) if x else None, V(wr) if wr else None, None,
                       V(ids) if ids else None, V(w) if w else None, V(ws) if ws else None,
                       nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(tokens=-1), lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(top_k=0), lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(top_k=9, experts=8), lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(top_k=17, experts=64), lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(experts=513), lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(hidden=100), lib.MOE_ERR_UNSUPPORTED),
    (dict(ffn=96), lib.MOE_ERR_UNSUPPORTED),
    (dict(hidden=192), lib.MOE_ERR_UNSUPPORTED),
    (dict(ffn=192), lib.MOE_ERR_UNSUPPORTED),
    (dict(act="f32", wdt="bf16"), lib.MOE_ERR_UNSUPPORTED),
    (dict(act="bf16", wdt="f32"), lib.MOE_ERR_UNSUPPORTED),
    (dict(act="f32", wdt="nvfp4"), lib.MOE_ERR_UNSUPPORTED),
    (dict(act="f32", wdt="mxfp8"), lib.MOE_ERR_UNSUPPORTED),
    (dict(wdt="mxfp8", hidden=256, ffn=512), lib.MOE_ERR_UNSUPPORTED),
    (dict(wdt="mxfp8", hidden=512, ffn=256), lib.MOE_ERR_UNSUPPORTED),
    (dict(wdt="mxfp4", hidden=256, ffn=512), lib.MOE_ERR_UNSUPPORTED),
    (dict(act="f32", wdt="mxfp4"), lib.MOE_ERR_UNSUPPORTED),
])
def test_problem_validation(L, kw, status):
    base = dict(tokens=16, hidden=256, experts=8, top_k=2, ffn=128, act="bf16", wdt="bf16")
    base.update(kw)
    p = lib.problem(**base)
    assert _call_route(L, p) == status
    n = C.c_size_t()
    assert L.moe_workspace_size(C.byref(p), C.byref(n)) == status


def test_pointer_validation(L):
    p = lib.problem(16, 256, 8, 2, 128)
    assert _call_route(L, p, x=0) == lib.MOE_ERR_INVALID_ARGUMENT
    assert _call_route(L, p, ids=0) == lib.MOE_ERR_INVALID_ARGUMENT
    assert _call_route(L, p, x=FAKE + 2) == lib.MOE_ERR_INVALID_ARGUMENT  # misaligned
    assert _call_route(L, p, ws=0) == lib.MOE_ERR_INVALID_ARGUMENT
    assert _call_route(L, p, nbytes=100) == lib.MOE_ERR_WORKSPACE_TOO_SMALL


def test_gemm_and_forward_validation(L):
    V = C.c_void_p
    p = lib.problem(16, 256, 8, 2, 128, wdt="nvfp4")
    w = lib.ExpertWeights(FAKE, FAKE, None, None, None, None, 0)  # NVFP4 without scales
    assert L.moe_grouped_gemm(C.byref(p), 0, V(FAKE), None, V(FAKE), C.byref(w), V(FAKE), V(FAKE),
                              1 << 40, None) == lib.MOE_ERR_INVALID_ARGUMENT
    w = lib.ExpertWeights(FAKE, FAKE, FAKE, FAKE, None, None, 0)
    assert L.moe_grouped_gemm(C.byref(p), 7, V(FAKE), None, V(FAKE), C.byref(w), V(FAKE), V(FAKE),
                              1 << 40, None) == lib.MOE_ERR_INVALID_ARGUMENT  # bad kind
    assert L.moe_grouped_gemm(C.byref(p), 1, V(FAKE), V(FAKE), V(FAKE), C.byref(w), V(FAKE),
                              V(FAKE), 1 << 40, None) == lib.MOE_ERR_INVALID_ARGUMENT  # down + gather
    assert L.moe_forward(C.byref(p), V(FAKE), V(FAKE), None, C.byref(w), V(FAKE), None, None, None,
                         None, None, None, V(FAKE), 10, None) == lib.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_combine(C.byref(p), None, V(FAKE), V(FAKE), V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    # layouts: bf16 weights row-major or packed, nothing else; NVFP4 weights row-major or, where
    # the shape tiles (H % 256, F % 128), packed; fp32 weights row-major only
    pb = lib.problem(16, 256, 8, 2, 128, wdt="bf16")
    for layout, status in ((0, lib.MOE_ERR_WORKSPACE_TOO_SMALL), (1, lib.MOE_ERR_WORKSPACE_TOO_SMALL),
                           (2, lib.MOE_ERR_INVALID_ARGUMENT), (-1, lib.MOE_ERR_INVALID_ARGUMENT)):
        wb = lib.ExpertWeights(FAKE, FAKE, None, None, None, None, layout)
        assert L.moe_forward(C.byref(pb), V(FAKE), V(FAKE), None, C.byref(wb), V(FAKE), None, None,
                             None, None, None, None, V(FAKE), 10, None) == status
    p192 = lib.problem(16, 192, 8, 2, 128, wdt="nvfp4")
    for layout, status in ((1, lib.MOE_ERR_UNSUPPORTED), (2, lib.MOE_ERR_INVALID_ARGUMENT)):
        w = lib.ExpertWeights(FAKE, FAKE, FAKE, FAKE, None, None, layout)
        assert L.moe_forward(C.byref(p192), V(FAKE), V(FAKE), None, C.byref(w), V(FAKE), None, None,
                             None, None, None, None, V(FAKE), 1 << 40, None) == status
    pf32 = lib.problem(16, 256, 8, 2, 128, act="f32", wdt="f32")
    for layout, status in ((0, lib.MOE_ERR_WORKSPACE_TOO_SMALL), (1, lib.MOE_ERR_INVALID_ARGUMENT)):
        wf = lib.ExpertWeights(FAKE, FAKE, None, None, None, None, layout)
        assert L.moe_forward(C.byref(pf32), V(FAKE), V(FAKE), None, C.byref(wf), V(FAKE), None, None,
                             None, None, None, None, V(FAKE), 10, None) == status
    pmx = lib.problem(16, 512, 8, 2, 512, wdt="mxfp8")
    for layout in (0, 1):  # MX codes row-major or packed
        wm = lib.ExpertWeights(FAKE, FAKE, FAKE, FAKE, None, None, layout)
        assert L.moe_forward(C.byref(pmx), V(FAKE), V(FAKE), None, C.byref(wm), V(FAKE), None, None,
                             None, None, None, None, V(FAKE), 10, None) == lib.MOE_ERR_WORKSPACE_TOO_SMALL
    w = lib.ExpertWeights(FAKE, FAKE, FAKE, FAKE, None, None, 1)  # packed NVFP4 is validated
    assert L.moe_forward(C.byref(p), V(FAKE), V(FAKE), None, C.byref(w), V(FAKE), None, None, None,
                         None, None, None, V(FAKE), 10, None) == lib.MOE_ERR_WORKSPACE_TOO_SMALL
    # packing: not for fp32 weights, no aliasing, shapes the layout can tile
    pf = lib.problem(16, 256, 8, 2, 128, act="f32", wdt="f32")
    assert L.moe_pack_weights(C.byref(pf), V(FAKE), V(FAKE), V(FAKE + 4096), V(FAKE + 8192),
                              None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_pack_weights(C.byref(p192), V(FAKE), None, V(FAKE + 4096), None,
                              None) == lib.MOE_ERR_UNSUPPORTED
    # NVFP4 scales: NVFP4 only, pairs, no aliasing, alignment, shapes the layout can tile
    ps = L.moe_pack_scales
    assert ps(C.byref(pb), V(FAKE), None, V(FAKE + 4096), None, None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert ps(C.byref(p), V(FAKE), None, None, None, None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert ps(C.byref(p), V(FAKE), None, V(FAKE), None, None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert ps(C.byref(p), V(FAKE + 4), None, V(FAKE + 4096), None, None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert ps(C.byref(p192), V(FAKE), None, V(FAKE + 4096), None, None) == lib.MOE_ERR_UNSUPPORTED
    assert ps(C.byref(p), None, None, None, None, None) == lib.MOE_OK  # nothing to pack
    a, b = lib.packed_weights_size(p)
    assert a == 8 * 2 * 128 * 128 and b == 8 * 256 * 64  # NVFP4 bytes, two values per byte
    with pytest.raises(lib.MoeError):
        lib.packed_weights_size(p192)
    assert L.moe_pack_weights(C.byref(pb), V(FAKE), None, V(FAKE), None, None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_pack_weights(C.byref(lib.problem(16, 192, 8, 2, 128)), V(FAKE), None, V(FAKE + 4096),
                              None, None) == lib.MOE_ERR_UNSUPPORTED


def test_mxfp8_validation(L):
    V = C.c_void_p
    p = lib.problem(16, 512, 8, 2, 512, wdt="mxfp8")
    w = lib.ExpertWeights(FAKE, FAKE, None, None, None, None, 0)  # MXFP8 without scales
    assert L.moe_forward(C.byref(p), V(FAKE), V(FAKE), None, C.byref(w), V(FAKE), None, None, None,
                         None, None, None, V(FAKE), 1 << 40, None) == lib.MOE_ERR_INVALID_ARGUMENT
    w = lib.ExpertWeights(FAKE, FAKE, FAKE, FAKE, None, None, 3)  # no such layout
    assert L.moe_forward(C.byref(p), V(FAKE), V(FAKE), None, C.byref(w), V(FAKE), None, None, None,
                         None, None, None, V(FAKE), 1 << 40, None) == lib.MOE_ERR_INVALID_ARGUMENT
    a, b = lib.packed_weights_size(p)
    assert a == 8 * 2 * 512 * 512 and b == 8 * 512 * 512  # one byte per code
    a, b = lib.packed_weights_size(lib.problem(16, 512, 8, 2, 512, wdt="mxfp4"))
    assert a == 8 * 2 * 512 * 256 and b == 8 * 512 * 256  # two codes per byte
    q = L.moe_quantize_mxfp8
    assert q(V(FAKE), 4, 48, V(FAKE), V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT    # K % 32
    assert q(V(FAKE), -1, 64, V(FAKE), V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert q(V(FAKE + 8), 4, 64, V(FAKE), V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert q(V(FAKE), 4, 64, None, V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert q(None, 0, 64, None, None, None) == lib.MOE_OK                               # no rows


def test_probe_validation(L):
    V = C.c_void_p
    assert L.moe_probe_mfma_bf16(0, 1, V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_probe_mfma_bf16(1, 0, V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_probe_mfma_bf16(1, 1, None, None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_probe_read(V(FAKE), 0, V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_probe_read(V(FAKE), 100, V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_probe_read(V(FAKE + 8), 1024, V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_probe_read(None, 1024, V(FAKE), None) == lib.MOE_ERR_INVALID_ARGUMENT
    for bad in ((V(FAKE), 0, V(FAKE)), (V(FAKE), 100, V(FAKE)), (V(FAKE + 8), 1024, V(FAKE)),
                (None, 1024, V(FAKE))):
        assert L.moe_probe_read_nt(*bad, None) == lib.MOE_ERR_INVALID_ARGUMENT


def test_grouped_gemm_timing_probe_validation(L):
    """moe_probe_grouped_gemm_times checks its own arguments (launches, the host time array, the
    flush buffer) before any HIP call, and with no tokens fills the times with zeros."""
    V = C.c_void_p
    p = lib.problem(16, 256, 8, 2, 128)
    w = lib.ExpertWeights(FAKE, FAKE, None, None, None, None, 1)
    ms = (C.c_float * 4)(7.0, 7.0, 7.0, 7.0)
    f = L.moe_probe_grouped_gemm_times
    args = lambda kind=0, launches=4, times=ms, fb=None, fn=0, fo=None, prob=p: (
        C.byref(prob), kind, V(FAKE), None, V(FAKE), C.byref(w), V(FAKE), V(FAKE), 1 << 40, fb, fn,
        fo, launches, times, None)
    assert f(*args(launches=0)) == lib.MOE_ERR_INVALID_ARGUMENT
    assert f(*args(launches=100001)) == lib.MOE_ERR_INVALID_ARGUMENT
    assert f(*args(times=None)) == lib.MOE_ERR_INVALID_ARGUMENT
    assert f(*args(kind=2)) == lib.MOE_ERR_INVALID_ARGUMENT
    assert f(*args(fb=None, fn=1024, fo=V(FAKE))) == lib.MOE_ERR_INVALID_ARGUMENT       # no buffer
    assert f(*args(fb=V(FAKE), fn=100, fo=V(FAKE))) == lib.MOE_ERR_INVALID_ARGUMENT     # not x16
    assert f(*args(fb=V(FAKE + 8), fn=1024, fo=V(FAKE))) == lib.MOE_ERR_INVALID_ARGUMENT
    assert f(*args(fb=V(FAKE), fn=1024, fo=None)) == lib.MOE_ERR_INVALID_ARGUMENT
    empty = lib.problem(0, 256, 8, 2, 128)
    assert f(*args(prob=empty)) == lib.MOE_OK
    assert list(ms) == [0.0] * 4
