"""Device-resident MoE layer: torch owns the buffers, the C ABI does every step.

``MoELayer`` uploads a set of host arrays (as produced by ``synth``) into torch device
tensors, sizes the workspace with ``moe_workspace_size`` and calls ``moe_forward`` (or the
stage entry points) on torch's current stream.  Nothing here computes any part of the layer.
"""
from __future__ import annotations

import numpy as np
import torch

from . import lib

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(a: np.ndarray | None, device, kind: str | None = None):
    """Host array -> device tensor.  ``kind='bf16'`` reinterprets uint16 bit patterns."""
    if a is None:
        return None
    if kind == "bf16" or (a.dtype == np.uint16 and kind is None):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array (bf16 becomes uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class MoELayer:
    def __init__(self, tokens, hidden, experts, top_k, ffn, act, wdt, inputs: dict,
                 device="cuda:0", renormalize=True, path="auto", expert_begin=0, local_experts=0,
                 weight_layout="packed"):
        """``inputs`` holds the weights of the held experts only when ``local_experts`` is set
        (expert parallelism: experts [expert_begin, expert_begin + local_experts)).  bf16 and MX
        weights, and NVFP4 bytes and scales, are packed once (moe_pack_weights /
        moe_pack_scales) when ``weight_layout`` is "packed" and the shape allows it (NVFP4:
        H % 256 == 0, F % 128 == 0), else handed to the library row-major."""
        self.device = torch.device(device)
        self.T, self.H, self.E, self.k, self.F = tokens, hidden, experts, top_k, ffn
        self.act, self.wdt = act, wdt
        self.renormalize, self.path = renormalize, path
        self.expert_begin, self.local_experts = expert_begin, local_experts
        self.problem = self.problem_for(tokens)
        d = self.device
        self.w_router = to_device(inputs["w_router"], d, "bf16" if act == "bf16" else None)
        self.bias = to_device(inputs.get("bias"), d)
        wk = "bf16" if wdt == "bf16" else None
        self.w13 = to_device(inputs["w13"], d, wk)
        self.w2 = to_device(inputs["w2"], d, wk)
        layout = lib.LAYOUT_ROW_MAJOR
        if wdt in ("bf16", "mxfp8", "mxfp4") and weight_layout == "packed":
            p13 = torch.empty_like(self.w13)
            p2 = torch.empty_like(self.w2)
            lib.pack_weights(self.problem, self.w13, self.w2, p13, p2)
            torch.cuda.current_stream(d).synchronize()
            self.w13, self.w2 = p13, p2
            layout = lib.LAYOUT_PACKED
        self.w13_scale = to_device(inputs.get("w13_scale"), d)
        self.w2_scale = to_device(inputs.get("w2_scale"), d)
        if wdt == "nvfp4" and weight_layout == "packed" and hidden % 256 == 0 and ffn % 128 == 0:
            tensors = (self.w13, self.w2, self.w13_scale, self.w2_scale)
            p13, p2, s13, s2 = (torch.empty_like(t) for t in tensors)
            lib.pack_weights(self.problem, self.w13, self.w2, p13, p2)
            lib.pack_scales(self.problem, self.w13_scale, self.w2_scale, s13, s2)
            torch.cuda.current_stream(d).synchronize()
            self.w13, self.w2, self.w13_scale, self.w2_scale = p13, p2, s13, s2
            layout = lib.LAYOUT_PACKED
        self.layout = layout
        self.w13_gscale = to_device(inputs.get("w13_gscale"), d)
        self.w2_gscale = to_device(inputs.get("w2_gscale"), d)
        self.weights = lib.weights(self.w13, self.w2, self.w13_scale, self.w2_scale,
                                   self.w13_gscale, self.w2_gscale, layout)
        self._ws_tokens = -1
        self.ws = None

    @classmethod
    def from_workload(cls, wl, inputs, device="cuda:0", path="auto", expert_begin=0,
                      local_experts=0, weight_layout="packed"):
        return cls(wl.tokens, wl.hidden, wl.experts, wl.top_k, wl.ffn, wl.act, wl.wdt, inputs,
                   device=device, renormalize=wl.renormalize, path=path,
                   expert_begin=expert_begin, local_experts=local_experts,
                   weight_layout=weight_layout)

    def problem_for(self, tokens: int, path: str | None = None):
        return lib.problem(tokens, self.H, self.E, self.k, self.F, self.act, self.wdt,
                           self.renormalize, path or self.path, self.expert_begin,
                           self.local_experts)

    def workspace(self, tokens: int, path: str | None = None) -> torch.Tensor:
        n = lib.workspace_size(self.problem_for(tokens, path))
        if self.ws is None or self.ws.numel() < n:
            self.ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        return self.ws

    def act_tensor(self, x: np.ndarray) -> torch.Tensor:
        return to_device(x, self.device, "bf16" if self.act == "bf16" else None)

    def empty_act(self, *shape):
        return torch.empty(*shape, dtype=_TORCH[self.act], device=self.device)

    def forward(self, x: torch.Tensor, debug: bool = False, path: str | None = None, y=None,
                stream=None):
        T = x.shape[0]
        p = self.problem_for(T, path)
        ws = self.workspace(T, path)
        y = self.empty_act(T, self.H) if y is None else y
        dbg = {}
        if debug:
            A, dev = T * self.k, self.device
            dbg = dict(topk_ids=torch.empty(T, self.k, dtype=torch.int32, device=dev),
                       topk_w=torch.empty(T, self.k, dtype=torch.float32, device=dev),
                       counts=torch.empty(self.E, dtype=torch.int32, device=dev),
                       offsets=torch.empty(self.E + 1, dtype=torch.int32, device=dev),
                       sorted_token=torch.empty(A, dtype=torch.int32, device=dev),
                       inv_perm=torch.empty(A, dtype=torch.int32, device=dev))
        lib.forward(p, x, self.w_router, self.bias, self.weights, y, ws, stream=stream, **dbg)
        return (y, dbg) if debug else y
