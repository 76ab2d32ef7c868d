"""Thin Python binding of the C ABI in ``include/moe.h`` (argument marshalling only).

Every entry point here calls the same-named C function of ``libmoe_mi355x.so`` with device
pointers taken from torch tensors and the hipStream_t of torch's current stream.  No step
of the layer runs in Python; if the library is missing this module raises at import time
of the first call instead of falling back to anything.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")

(MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_DEVICE,
 MOE_ERR_SCRATCH_TOO_SMALL) = range(6)
STATIC_SCRATCH_BYTES = 64 << 20  # MOE_STATIC_SCRATCH_BYTES
MOE_F32, MOE_BF16, MOE_NVFP4, MOE_MXFP8, MOE_MXFP4 = 0, 1, 2, 3, 4
GATE_UP_SWIGLU, DOWN = 0, 1
PATH_AUTO, PATH_PREFILL, PATH_DECODE, PATH_DECODE_FUSED = 0, 1, 2, 3
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "nvfp4": MOE_NVFP4, "mxfp8": MOE_MXFP8, "mxfp4": MOE_MXFP4}
PATHS = {"auto": PATH_AUTO, "prefill": PATH_PREFILL, "decode": PATH_DECODE, "fused": PATH_DECODE_FUSED}

#: every symbol the header declares
EXPORTS = ("moe_status_string", "moe_workspace_size", "moe_packed_weights_size", "moe_pack_weights",
           "moe_pack_scales", "moe_route", "moe_permute", "moe_grouped_gemm", "moe_combine", "moe_forward",
           "moe_quantize_mxfp8", "moe_probe_mfma_bf16", "moe_probe_read", "moe_probe_read_nt", "moe_forward_static",
           "moe_probe_grid_barrier", "moe_probe_grouped_gemm_times")
PROBE_SYNC_BYTES = 8256  # MOE_PROBE_SYNC_BYTES
LAYOUT_ROW_MAJOR, LAYOUT_PACKED = 0, 1


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))


class Problem(C.Structure):
    _fields_ = [("num_tokens", C.c_int32), ("hidden", C.c_int32), ("num_experts", C.c_int32),
                ("top_k", C.c_int32), ("ffn", C.c_int32), ("act_dtype", C.c_int32),
                ("w_dtype", C.c_int32), ("renormalize", C.c_int32), ("path", C.c_int32),
                ("expert_begin", C.c_int32), ("local_experts", C.c_int32)]


class ExpertWeights(C.Structure):
    _fields_ = [("w13", C.c_void_p), ("w2", C.c_void_p), ("w13_scale", C.c_void_p),
                ("w2_scale", C.c_void_p), ("w13_gscale", C.c_void_p), ("w2_gscale", C.c_void_p),
                ("layout", C.c_int32)]


_lock = threading.Lock()
_lib = None


def load() -> C.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libmoe_mi355x.so is not built (run "
                                   "`python -m mixture_experts_layer_softmax_amd.build`)")
            L = C.CDLL(LIB_PATH)
            vp, sz, i32 = C.c_void_p, C.c_size_t, C.c_int
            P = C.POINTER(Problem)
            L.moe_status_string.restype = C.c_char_p
            L.moe_status_string.argtypes = [i32]
            L.moe_workspace_size.restype = i32
            L.moe_workspace_size.argtypes = [P, C.POINTER(C.c_size_t)]
            L.moe_packed_weights_size.restype = i32
            L.moe_packed_weights_size.argtypes = [P, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]
            L.moe_pack_weights.restype = i32
            L.moe_pack_weights.argtypes = [P, vp, vp, vp, vp, vp]
            L.moe_pack_scales.restype = i32
            L.moe_pack_scales.argtypes = [P, vp, vp, vp, vp, vp]
            L.moe_route.restype = i32
            L.moe_route.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
            L.moe_permute.restype = i32
            L.moe_permute.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
            L.moe_grouped_gemm.restype = i32
            L.moe_grouped_gemm.argtypes = [P, i32, vp, vp, vp, C.POINTER(ExpertWeights), vp, vp, sz, vp]
            L.moe_combine.restype = i32
            L.moe_combine.argtypes = [P, vp, vp, vp, vp, vp]
            L.moe_quantize_mxfp8.restype = i32
            L.moe_quantize_mxfp8.argtypes = [vp, C.c_int64, C.c_int32, vp, vp, vp]
            L.moe_probe_mfma_bf16.restype = i32
            L.moe_probe_mfma_bf16.argtypes = [C.c_int32, C.c_int32, vp, vp]
            L.moe_probe_read.restype = i32
            L.moe_probe_read.argtypes = [vp, sz, vp, vp]
            L.moe_probe_read_nt.restype = i32
            L.moe_probe_read_nt.argtypes = [vp, sz, vp, vp]
            L.moe_probe_grid_barrier.restype = i32
            L.moe_probe_grid_barrier.argtypes = [C.c_int32, C.c_int32, vp, C.c_uint32, vp]
            L.moe_probe_grouped_gemm_times.restype = i32
            L.moe_probe_grouped_gemm_times.argtypes = [P, i32, vp, vp, vp, C.POINTER(ExpertWeights), vp,
                                                       vp, sz, vp, sz, vp, C.c_int32,
                                                       C.POINTER(C.c_float), vp]
            L.moe_forward.restype = i32
            L.moe_forward.argtypes = [P, vp, vp, vp, C.POINTER(ExpertWeights), vp, vp, vp, vp, vp,
                                      vp, vp, vp, sz, vp]
            L.moe_forward_static.restype = i32
            L.moe_forward_static.argtypes = [P, vp, vp, vp, C.POINTER(ExpertWeights), vp, vp, vp, vp,
                                             vp, vp, vp, vp]
            _lib = L
    return _lib


def status_string(s: int) -> str:
    return load().moe_status_string(int(s)).decode()


def problem(tokens, hidden, experts, top_k, ffn, act="bf16", wdt="bf16", renormalize=True,
            path="auto", expert_begin=0, local_experts=0) -> Problem:
    """``expert_begin``/``local_experts``: the held expert range under expert parallelism
    (0/0 = all experts)."""
    return Problem(int(tokens), int(hidden), int(experts), int(top_k), int(ffn), DTYPES[act],
                   DTYPES[wdt], int(bool(renormalize)), PATHS[path], int(expert_begin),
                   int(local_experts))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return C.c_void_p(int(stream))
    import torch

    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status, what):
    if status != MOE_OK:
        raise MoeError(status, what)


def workspace_size(p: Problem) -> int:
    n = C.c_size_t(0)
    _check(load().moe_workspace_size(C.byref(p), C.byref(n)), "moe_workspace_size")
    return n.value


def weights(w13, w2, w13_scale=None, w2_scale=None, w13_gscale=None, w2_gscale=None,
            layout=LAYOUT_ROW_MAJOR) -> ExpertWeights:
    return ExpertWeights(*[t.data_ptr() if t is not None else None
                           for t in (w13, w2, w13_scale, w2_scale, w13_gscale, w2_gscale)],
                         int(layout))


def packed_weights_size(p: Problem):
    a, b = C.c_size_t(0), C.c_size_t(0)
    _check(load().moe_packed_weights_size(C.byref(p), C.byref(a), C.byref(b)), "moe_packed_weights_size")
    return a.value, b.value


def pack_weights(p, w13, w2, w13_packed, w2_packed, stream=None):
    _check(load().moe_pack_weights(C.byref(p), _ptr(w13), _ptr(w2), _ptr(w13_packed),
                                   _ptr(w2_packed), _stream(stream)), "moe_pack_weights")


def pack_scales(p, w13_scale, w2_scale, w13_scale_packed, w2_scale_packed, stream=None):
    _check(load().moe_pack_scales(C.byref(p), _ptr(w13_scale), _ptr(w2_scale), _ptr(w13_scale_packed),
                                  _ptr(w2_scale_packed), _stream(stream)), "moe_pack_scales")


def route(p, x, w_router, bias, topk_ids, topk_w, ws, stream=None):
    _check(load().moe_route(C.byref(p), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(topk_ids),
                            _ptr(topk_w), _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream)), "moe_route")


def permute(p, topk_ids, counts, offsets, sorted_token, inv_perm, ws, x=None, x_perm=None,
            stream=None):
    _check(load().moe_permute(C.byref(p), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                              _ptr(sorted_token), _ptr(inv_perm), _ptr(x), _ptr(x_perm), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "moe_permute")


def grouped_gemm(p, kind, a, a_rows, offsets, w: ExpertWeights, out, ws, stream=None):
    _check(load().moe_grouped_gemm(C.byref(p), int(kind), _ptr(a), _ptr(a_rows), _ptr(offsets),
                                   C.byref(w), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "moe_grouped_gemm")


def combine(p, y_perm, inv_perm, topk_w, y, stream=None):
    _check(load().moe_combine(C.byref(p), _ptr(y_perm), _ptr(inv_perm), _ptr(topk_w), _ptr(y),
                              _stream(stream)), "moe_combine")


def forward(p, x, w_router, bias, w: ExpertWeights, y, ws, topk_ids=None, topk_w=None,
            counts=None, offsets=None, sorted_token=None, inv_perm=None, stream=None):
    _check(load().moe_forward(C.byref(p), _ptr(x), _ptr(w_router), _ptr(bias), C.byref(w), _ptr(y),
                              _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                              _ptr(sorted_token), _ptr(inv_perm), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "moe_forward")


def forward_static(p, x, w_router, bias, w: ExpertWeights, y, topk_ids=None, topk_w=None,
                   counts=None, offsets=None, sorted_token=None, inv_perm=None, stream=None):
    """moe_forward_static: the layer with the library's static per-GPU scratch (no workspace)."""
    _check(load().moe_forward_static(C.byref(p), _ptr(x), _ptr(w_router), _ptr(bias), C.byref(w),
                                     _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
                                     _ptr(offsets), _ptr(sorted_token), _ptr(inv_perm),
                                     _stream(stream)), "moe_forward_static")


def quantize_mxfp8(x, codes, scales, stream=None):
    """MXFP8 quantization of bf16 rows x [rows, K] into codes [rows, K] / scales [rows, K/32]."""
    rows, K = x.shape
    _check(load().moe_quantize_mxfp8(_ptr(x), int(rows), int(K), _ptr(codes), _ptr(scales),
                                     _stream(stream)), "moe_quantize_mxfp8")


def probe_mfma_bf16(blocks, iters, out, stream=None):
    """Launch the bf16 MFMA rate probe (moe_probe.h); returns its FLOP count."""
    _check(load().moe_probe_mfma_bf16(int(blocks), int(iters), _ptr(out), _stream(stream)),
           "moe_probe_mfma_bf16")
    return float(blocks) * 4 * iters * 8 * 16384


def probe_read(buf, out, stream=None, nontemporal=False):
    """Launch the HBM read-stream probe over all of ``buf`` (moe_probe_read, which evicts the
    caches, or with ``nontemporal`` moe_probe_read_nt); returns the bytes read."""
    n = buf.numel() * buf.element_size()
    name = "moe_probe_read_nt" if nontemporal else "moe_probe_read"
    _check(getattr(load(), name)(_ptr(buf), n, _ptr(out), _stream(stream)), name)
    return float(n)


def probe_grouped_gemm_times(p, kind, a, a_rows, offsets, w: ExpertWeights, out, ws, launches,
                             flush=None, flush_out=None, stream=None):
    """moe_probe_grouped_gemm_times: the GEMM of moe_grouped_gemm launched `launches` times, each
    bracketed by events (the tile-list kernel and the optional cache flush over all of `flush`
    outside the brackets); returns the per-launch times in ms (synchronizes the stream)."""
    ms = (C.c_float * int(launches))()
    nflush = 0 if flush is None else flush.numel() * flush.element_size()
    _check(load().moe_probe_grouped_gemm_times(C.byref(p), int(kind), _ptr(a), _ptr(a_rows),
                                               _ptr(offsets), C.byref(w), _ptr(out), _ptr(ws),
                                               ws.numel() * ws.element_size(), _ptr(flush), nflush,
                                               _ptr(flush_out), int(launches), ms, _stream(stream)),
           "moe_probe_grouped_gemm_times")
    return [float(v) for v in ms]


def probe_grid_barrier(blocks, barriers, sync, spin_limit=1 << 20, stream=None):
    """Launch `barriers` grid barriers of the single-launch decode kernel on `blocks` blocks."""
    _check(load().moe_probe_grid_barrier(int(blocks), int(barriers), _ptr(sync), int(spin_limit),
                                         _stream(stream)), "moe_probe_grid_barrier")
