"""Per-token brute force of the MoE layer for tiny inputs (numpy, fp64, no permutation).

Written independently of the oracle to pin it: it decodes weights with numpy/torch routines
and the published E2M1 table, selects experts with ``numpy.lexsort``, and evaluates each
token's experts directly (no dispatch, no combine buffers).  Router logits are taken as an
argument because their canonical fp32 order is pinned separately.
"""
import json
import os

import numpy as np
import torch

_GOLD = os.path.join(os.path.dirname(__file__), "golden", "ocp_formats.json")
E2M1_MAG = np.array(json.load(open(_GOLD))["e2m1_magnitudes_by_code"], dtype=np.float64)


def bf16_to_f64(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def act_f64(a):
    return a.astype(np.float64) if a.dtype == np.float32 else bf16_to_f64(a)


def e4m3_to_f64(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e2m1_to_f64(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAG[codes & 7]
    return np.where(codes & 8, -mag, mag)


def dense_weights(inputs, wdt):
    """W13[E,2F,H] and W2[E,H,F] as float64."""
    if wdt == "f32":
        return inputs["w13"].astype(np.float64), inputs["w2"].astype(np.float64)
    if wdt == "bf16":
        return bf16_to_f64(inputs["w13"]), bf16_to_f64(inputs["w2"])
    if wdt == "mxfp8":
        return tuple(e4m3_to_f64(inputs[w]) * np.repeat(np.exp2(inputs[s].astype(np.float64) - 127), 32, axis=2)
                     for w, s in (("w13", "w13_scale"), ("w2", "w2_scale")))
    if wdt == "mxfp4":
        out = []
        for w, s in (("w13", "w13_scale"), ("w2", "w2_scale")):
            p = inputs[w]
            codes = np.stack([p & 15, p >> 4], axis=-1).reshape(p.shape[0], p.shape[1], -1)
            out.append(e2m1_to_f64(codes) * np.repeat(np.exp2(inputs[s].astype(np.float64) - 127), 32, axis=2))
        return out[0], out[1]
    out = []
    for w, s, g in (("w13", "w13_scale", "w13_gscale"), ("w2", "w2_scale", "w2_gscale")):
        p = inputs[w]
        codes = np.stack([p & 15, p >> 4], axis=-1).reshape(p.shape[0], p.shape[1], -1)
        vals = e2m1_to_f64(codes)
        sc = np.repeat(e4m3_to_f64(inputs[s]), 16, axis=2)
        gs = inputs[g].astype(np.float64)[:, None, None]
        out.append(vals * sc * gs)
    return out[0], out[1]


# the 127 non-negative finite E4M3 values in code order (torch's float8_e4m3fn decode)
E4M3_POS = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def mx_round_trip(v):
    """MX quantization of a float64 vector (OCP MX v1.0: per 32 elements the E8M0 exponent
    X = floor(log2 amax) - 8, elements v / 2^X clamped to +-448 and rounded to the nearest E4M3
    value, ties to the even code), returned decoded."""
    b = np.asarray(v, dtype=np.float64).reshape(-1, 32)
    amax = np.abs(b).max(axis=1)
    X = np.full(amax.shape, -127.0)
    nz = amax > 0
    X[nz] = np.clip(np.floor(np.log2(amax[nz])) - 8, -127, 127)
    q = np.minimum(np.abs(b) * np.exp2(-X)[:, None], 448.0)
    hi = np.clip(np.searchsorted(E4M3_POS, q, side="left"), 1, 126)  # E4M3_POS[hi-1] < q <= E4M3_POS[hi]
    lo = hi - 1
    dl, dh = q - E4M3_POS[lo], E4M3_POS[hi] - q
    code = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(q == 0, 0, code)
    return (np.copysign(E4M3_POS[code], b) * np.exp2(X)[:, None]).reshape(np.shape(v))


def select(logits, k, renormalize=True):
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        ids[t] = order[:k]
        l = logits[t].astype(np.float64)
        m = l.max()
        p = np.exp(l - m)
        p = p / p.sum()
        sel = p[ids[t]]
        w[t] = sel / sel.sum() if renormalize else sel
    return ids, w


def layer(inputs, logits, k, wdt, renormalize=True, keep=None):
    """y[T,H] in fp64, one token at a time.  ``keep(e)`` (optional) limits the sum to the
    experts it accepts (one rank's share under expert parallelism)."""
    x = act_f64(inputs["x"])
    w13, w2 = dense_weights(inputs, wdt)
    F = w2.shape[2]
    ids, w = select(logits, k, renormalize)
    y = np.zeros_like(x)
    if wdt in ("mxfp8", "mxfp4"):  # the layer quantizes its activations before each projection
        x = np.stack([mx_round_trip(r) for r in x])
    for t in range(x.shape[0]):
        for j in range(k):
            e = ids[t, j]
            if keep is not None and not keep(e):
                continue
            g = w13[e, :F] @ x[t]
            u = w13[e, F:] @ x[t]
            h = g / (1.0 + np.exp(-g)) * u
            if wdt in ("mxfp8", "mxfp4"):  # hid, a bf16 activation, rounded to bf16 and MX-quantized
                m, ex = np.frexp(h)
                h = mx_round_trip(np.ldexp(np.rint(m * 256.0) / 256.0, ex))
            y[t] += w[t, j] * (w2[e] @ h)
    return y, ids, w
