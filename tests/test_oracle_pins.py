"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test ties one oracle step to something other than the oracle itself: the published
format tables, library routines (torch's bf16 / float8 casts, numpy sorts and matmuls,
scipy's softmax), hand-derived values of the canonical router order, closed forms,
invariants of the layer's definition, and the per-token brute force in ``bruteforce.py``.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import bruteforce as BF
from mixture_experts_layer_softmax_amd import synth
from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    O.build()


# ---------------------------------------------------------------------------------------
# codecs
# ---------------------------------------------------------------------------------------

def test_bf16_decoder_matches_torch_on_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.decode_bf16(bits)
    ref = BF.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_decoder_matches_torch_and_spec_points():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3(codes)
    ref = BF.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    spec = json.load(open(os.path.join(GOLD, "ocp_formats.json")))
    for c, v in spec["e4m3_points"].items():
        got = O.decode_e4m3(np.array([int(c, 16)], np.uint8))[0]
        assert got == v and math.copysign(1, got) == math.copysign(1, v), c
    for c in spec["e4m3_nan_codes"]:
        assert np.isnan(O.decode_e4m3(np.array([int(c, 16)], np.uint8))[0])


def test_e2m1_decoder_matches_spec_table():
    spec = json.load(open(os.path.join(GOLD, "ocp_formats.json")))["e2m1_magnitudes_by_code"]
    codes = np.arange(16, dtype=np.uint8)
    got = O.decode_e2m1(codes)
    assert list(got[:8]) == spec
    assert list(-got[8:]) == spec
    assert np.signbit(got[8])  # code 0b1000 is negative zero


def test_e8m0_decoder_is_a_power_of_two_per_code():
    """OCP MX v1.0 scale format: code c stands for 2^(c - 127); 255 is NaN."""
    d = O.decode_e8m0(np.arange(256, dtype=np.uint8))
    assert np.array_equal(d[:255], np.exp2(np.arange(255) - 127.0)) and np.isnan(d[255])


def test_mx_quantizer_hand_values():
    """Blocks worked by hand from the OCP MX definition (shared exponent floor(log2 amax) - 8,
    E4M3 elements clamped to 448, nearest even)."""
    def q(first, rest=0.0):
        v = np.full(32, rest)
        v[0] = first
        c, sc, d = O.mx_quantize(v)
        return int(c[0]), int(sc[0]), float(d[0])
    assert q(1.0) == (0x78, 119, 1.0)            # 1.0 / 2^-8 = 256 = E4M3 0.1111.000
    assert q(1.75) == (0x7E, 119, 1.75)          # 448: the largest E4M3 value
    assert q(1.99)[:2] == (0x7E, 119)            # 509 clamps to 448
    assert q(-3.0) == (0x80 | 0x78 | 0x04, 120, -3.0)  # 384 = 1.5 * 2^8 -> 0.1111.100, sign bit
    c, sc, d = O.mx_quantize(np.zeros(32))
    assert np.all(c == 0) and sc[0] == 0 and np.all(d == 0)
    # 1 + 1/16 scales to 272, halfway between 256 (code 0x78, even) and 288 (0x79): ties to even
    v = np.zeros(32)
    v[0], v[1] = 1.0, 1.0625
    c, _, _ = O.mx_quantize(v)
    assert c[1] == 0x78
    v[1] = 1.0625 + 2.0 ** -40                   # just above the midpoint
    assert O.mx_quantize(v)[0][1] == 0x79


@pytest.mark.parametrize("wdt", ["mxfp8", "mxfp4"])
def test_mx_down_projection_quantizes_the_bf16_hid(wdt):
    """The MX layer's down projection quantizes hid as the layer's bf16 activation (the same
    input moe_quantize_mxfp8 takes), not the exact value.  Hand-worked: a block whose only
    non-zero element is 272.5 has amax in [256, 512), so X = 0.  Exactly, 272.5 lies above the
    E4M3 midpoint 272 of 256 and 288 and rounds to 288 (code 0x79); rounded to bf16 first (8
    significant bits, step 2 at 2^8) it becomes 272, the midpoint itself, which goes to the
    even code 0x78 = 256.  With W2 one-hot (MXFP8: 1.0 = E4M3 256 (0x78) at scale 2^-8; MXFP4:
    E2M1 4.0 (code 6) at scale 2^-2) the quantized hid element reads straight back as the output."""
    H = F = 64
    w = np.zeros((H, F), np.float32)
    w[np.arange(H), np.arange(H)] = 1.0                # y[h] = MX(hid)[h]
    if wdt == "mxfp8":
        codes, scales = synth.quantize_mxfp8(w)
        assert codes[0, 0] == 0x78 and scales[0, 0] == 119
    else:
        codes, scales = synth.quantize_mxfp4(w)
        assert codes[0, 0] & 15 == 6 and scales[0, 0] == 125
    inputs = dict(w2=codes[None], w2_scale=scales[None])
    hid = np.zeros((2, F))
    hid[0, 0] = 272.5                                  # the reading decides this code
    hid[1, 0] = 272.0 + 2.0 ** -20                     # both readings: bf16 272 -> 256 as well
    hid[:, 32] = 3.0                                   # second block: exactly representable
    y = O.down_rows(inputs, wdt, H, hid, np.zeros(2, np.int32))
    assert y[0, 0] == 256.0 and y[1, 0] == 256.0
    assert np.all(y[:, 32] == 3.0)
    rest = np.ones(H, bool)
    rest[[0, 32]] = False
    assert np.all(y[:, rest] == 0.0)
    # the exact value would have given 288: what the quantizer does to the unrounded 272.5
    assert O.mx_quantize(np.r_[272.5, np.zeros(31)])[2][0] == 288.0


def test_mx_quantizer_matches_numpy_reference_on_wide_ranges():
    rng = np.random.default_rng(21)
    n = 32 * 512
    v = rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))  # small elements underflow
    v[:32] = 0.0                                                   # an all-zero block
    v[32:64] = -0.0
    v[64:96] = np.exp2(rng.integers(-5, 5, 32).astype(float))      # amax exactly a power of two
    v[96:128] = (rng.integers(0, 16, 32) * 2 + 1) * 2.0 ** -5      # many midpoints of the E4M3 grid
    _, _, dec = O.mx_quantize(v)
    assert np.array_equal(dec, BF.mx_round_trip(v))
    c, sc, _ = O.mx_quantize(v)
    assert np.all(c[32:64] == 0x80)                                # -0 keeps its sign
    # each normal, unclamped element is within half an E4M3 step (1/16 relative); clamped ones
    # (scaled into (448, 512)) are set to 448 exactly
    scaled = np.abs(v) * np.exp2(-(sc.repeat(32).astype(float) - 127))
    normal = (scaled >= 2.0 ** -6) & (scaled <= 448)
    assert np.all(np.abs(dec - v)[normal] <= np.abs(v)[normal] / 16)
    clamped = scaled > 448
    assert clamped.any() and np.all(np.abs(dec[clamped]) == 448 * np.exp2(sc.repeat(32)[clamped] - 127.0))


def test_mx_quantizer_is_idempotent_and_matches_the_generator():
    rng = np.random.default_rng(22)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    c, sc, dec = O.mx_quantize(w.astype(np.float64))
    c2, sc2, dec2 = O.mx_quantize(dec)
    assert np.array_equal(c, c2) and np.array_equal(sc, sc2) and np.array_equal(dec, dec2)
    gc, gs = synth.quantize_mxfp8(w)
    assert np.array_equal(gc, c) and np.array_equal(gs, sc)


def test_mxfp4_encoding_hand_values_and_round_trip():
    """OCP MX v1.0 with E2M1 elements: shared exponent floor(log2 amax) - 2, elements clamped to
    6 and rounded to the nearest E2M1 value (ties to even); checked against hand-worked blocks and
    the per-element error bound, decoded with the brute force's own E2M1 table."""
    def enc(first, rest=0.0):
        w = np.full((1, 32), rest, dtype=np.float32)
        w[0, 0] = first
        packed, sc = synth.quantize_mxfp4(w)
        return int(packed[0, 0] & 15), int(sc[0, 0])
    assert enc(1.0) == (6, 125)        # 1.0 / 2^-2 = 4 = E2M1 code 6
    assert enc(1.5) == (7, 125)        # 6: the largest E2M1 value
    assert enc(1.9) == (7, 125)        # 7.6 clamps to 6
    assert enc(-0.75) == (8 | 7, 124)  # amax 0.75 -> X = -3, -0.75 / 2^-3 = -6
    assert enc(0.0) == (0, 0)          # all-zero block
    rng = np.random.default_rng(23)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    packed, sc = synth.quantize_mxfp4(w)
    codes = np.stack([packed & 15, packed >> 4], axis=-1).reshape(64, 256)
    X = np.repeat(sc.astype(np.float64) - 127, 32, axis=1)
    dec = BF.e2m1_to_f64(codes) * np.exp2(X)
    scaled = np.abs(w) * np.exp2(-X)
    normal = (scaled >= 1.0) & (scaled <= 6.0)      # E2M1 normals: one mantissa bit
    assert np.all(np.abs(dec - w)[normal] <= np.abs(w)[normal] / 4 + 1e-12)
    assert np.all(np.abs(dec - w)[scaled < 1.0] <= 0.25 * np.exp2(X)[scaled < 1.0] + 1e-12)
    assert np.all(np.abs(dec)[scaled > 6.0] == 6.0 * np.exp2(X)[scaled > 6.0])


def test_generator_bf16_rounding_matches_torch():
    a = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    a[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]  # exact ties go to even
    ours = synth.to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------------------
# canonical router logits
# ---------------------------------------------------------------------------------------

def _bf16(v):
    return synth.to_bf16_bits(np.asarray(v, dtype=np.float32))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_logits_exact_on_integer_inputs(act):
    """Small integers: every product and partial sum is exact in fp32, so the canonical
    order must return the exact integer dot product; a dropped or misplaced element shows."""
    rng = np.random.default_rng(1)
    T, E, H = 5, 7, 4096
    x = rng.integers(-8, 9, size=(T, H)).astype(np.float32)
    w = rng.integers(-8, 9, size=(E, H)).astype(np.float32)
    b = rng.integers(-100, 100, size=E).astype(np.float32)
    exact = x.astype(np.int64) @ w.astype(np.int64).T + b.astype(np.int64)
    cv = (lambda a: a) if act == "f32" else _bf16
    got = O.router_logits(cv(x), cv(w), b)
    assert np.array_equal(got.astype(np.int64), exact)


def test_logits_one_hot_picks_each_weight():
    rng = np.random.default_rng(2)
    E, H = 6, 1024
    w = _bf16(rng.standard_normal((E, H)) * 0.02)
    hs = np.arange(0, H, 37)
    x = np.zeros((hs.size, H), np.float32)
    x[np.arange(hs.size), hs] = 1.0
    got = O.router_logits(_bf16(x), w)
    assert np.array_equal(got, BF.bf16_to_f64(w)[:, hs].T.astype(np.float32))


def _products_case(prod: dict, H: int):
    """x = 1 everywhere a product is planted, w = the planted product (both exact)."""
    x = np.zeros((1, H), np.float32)
    w = np.zeros((1, H), np.float32)
    for h, v in prod.items():
        x[0, h] = 1.0
        w[0, h] = v
    return x, w


def test_canonical_order_chunks_of_a_partial_fold_first():
    """Hand-derived.  Products: 2^24 at h=0 (chunk 0 -> partial 0), -2^24 at h=8 (chunk 1 ->
    partial 1), +1 at h=512 (chunk 64 -> partial 0 again).  Partial 0 = fl(2^24 + 1) = 2^24
    (the tie rounds to even), partial 1 = -2^24, the fold gives 0.  A plain left-to-right sum
    would give 1, and the exact value is 1."""
    x, w = _products_case({0: 2.0 ** 24, 8: -(2.0 ** 24), 512: 1.0}, 520)
    assert O.router_logits(x, w)[0, 0] == 0.0
    assert O.router_logits(_bf16(x), _bf16(w))[0, 0] == 0.0


def test_canonical_order_fold_pairs_p_with_p_plus_off():
    """Hand-derived.  Partial 0 = 2^24, partial 1 = 1, partial 32 = -2^24 (chunks 0, 1, 32).
    The first fold (off = 32) cancels partials 0 and 32 exactly, the last one adds partial 1:
    result 1.  Folding the partials left to right would give fl(2^24 + 1) - 2^24 = 0."""
    x, w = _products_case({0: 2.0 ** 24, 8: 1.0, 256: -(2.0 ** 24)}, 512)
    assert O.router_logits(x, w)[0, 0] == 1.0


def test_canonical_order_fma_is_fused_per_element():
    """Hand-derived.  Element 0: x = w = 1 + 2^-12; fma onto +0 gives the rounded product
    1 + 2^-11 (its 2^-24 tail is a tie that rounds to even).  Element 1: x = 1 + 2^-12,
    w = -(1 + 2^-12); fma onto 1 + 2^-11 leaves exactly -2^-24.  A separately rounded product
    would leave 0, so the value pins one fused operation per element."""
    H = 8
    x = np.zeros((1, H), np.float32)
    w = np.zeros((1, H), np.float32)
    x[0, 0] = w[0, 0] = 1 + 2.0 ** -12
    x[0, 1] = 1 + 2.0 ** -12
    w[0, 1] = -(1 + 2.0 ** -12)
    assert O.router_logits(x, w)[0, 0] == -(2.0 ** -24)


def test_logits_within_higham_bound_of_fp64_dot():
    rng = np.random.default_rng(3)
    T, E, H = 16, 32, 4096
    x = _bf16(rng.standard_normal((T, H)))
    w = _bf16(rng.standard_normal((E, H)) * 0.02)
    b = rng.standard_normal(E).astype(np.float32)
    got = O.router_logits(x, w, b).astype(np.float64)
    xd, wd = BF.bf16_to_f64(x), BF.bf16_to_f64(w)
    exact = xd @ wd.T + b.astype(np.float64)
    n = H // 64 + 6 + 1
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    bound = gamma * (np.abs(xd) @ np.abs(wd).T + np.abs(b))
    assert np.all(np.abs(got - exact) <= bound)


def test_logits_zero_tokens_give_bias_exactly():
    w = _bf16(np.random.default_rng(4).standard_normal((9, 256)))
    b = np.random.default_rng(5).standard_normal(9).astype(np.float32)
    got = O.router_logits(np.zeros((3, 256), np.uint16), w, b)
    assert np.array_equal(got, np.broadcast_to(b, (3, 9)))


# ---------------------------------------------------------------------------------------
# selection and weights
# ---------------------------------------------------------------------------------------

def test_select_matches_lexsort_with_many_ties():
    rng = np.random.default_rng(6)
    logits = rng.integers(-3, 4, size=(500, 16)).astype(np.float32) * 0.5
    for k in (1, 2, 5, 16):
        ids, w = O.select(logits, k)
        bids, bw = BF.select(logits, k)
        assert np.array_equal(ids, bids)
        np.testing.assert_allclose(w, bw, rtol=1e-12, atol=0)


def test_select_exhaustive_ties_e4_k2():
    grid = np.array(np.meshgrid(*[[0.0, 1.0, 2.0]] * 4, indexing="ij")).reshape(4, -1).T
    logits = grid.astype(np.float32)
    ids, _ = O.select(logits, 2)
    bids, _ = BF.select(logits, 2)
    assert np.array_equal(ids, bids)


def test_select_all_equal_and_k_equals_e():
    ids, w = O.select(np.full((3, 8), 0.25, np.float32), 3)
    assert (ids == [0, 1, 2]).all() and np.allclose(w, 1 / 3, rtol=0, atol=1e-15)
    lg = np.random.default_rng(7).standard_normal((4, 8)).astype(np.float32)
    ids, w = O.select(lg, 8)
    assert np.array_equal(np.sort(ids, axis=1), np.tile(np.arange(8), (4, 1)))
    assert np.array_equal(ids, np.argsort(-lg, axis=1, kind="stable"))


def test_negative_zero_ties_with_positive_zero():
    lg = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert O.select(lg, 1)[0][0, 0] == 0


def test_weights_closed_forms():
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((200, 32)).astype(np.float32) * 2
    _, w = O.select(lg, 8)
    assert np.all(np.abs(w.sum(1) - 1) <= 1e-12)
    ids, w2 = O.select(lg, 2)
    l0 = lg[np.arange(200), ids[:, 0]].astype(np.float64)
    l1 = lg[np.arange(200), ids[:, 1]].astype(np.float64)
    np.testing.assert_allclose(w2[:, 0], scipy.special.expit(l0 - l1), rtol=1e-13)
    ids, wf = O.select(lg, 4, renormalize=False)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(wf, np.take_along_axis(full, ids, 1), rtol=1e-12)


# ---------------------------------------------------------------------------------------
# dispatch permutation
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (1000, 128, 8), (3, 256, 8), (0, 4, 2)])
def test_permutation_is_the_stable_counting_sort(T, E, k):
    rng = np.random.default_rng(9)
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    counts, offsets, st, ip = O.permute(ids, E)
    flat = ids.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(offsets[1:], np.cumsum(counts))
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(st, order // k)
    assert np.array_equal(np.sort(ip), np.arange(T * k))
    assert np.array_equal(st[ip], np.arange(T * k) // k)
    assert np.array_equal(ip[order], np.arange(T * k))


def test_permute_then_unpermute_is_identity():
    rng = np.random.default_rng(10)
    T, E, k, H = 100, 16, 4, 24
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = rng.standard_normal((T, H))
    _, _, st, ip = O.permute(ids, E)
    x_perm = x[st]
    back = x_perm[ip].reshape(T, k, H)
    for j in range(k):
        assert np.array_equal(back[:, j], x)


@pytest.mark.parametrize("b,n", [(0, 128), (0, 32), (32, 32), (96, 32), (5, 1), (127, 1)])
def test_held_dispatch_is_the_stable_sort_restricted_to_held_experts(b, n):
    """Expert parallelism: the dispatch of a held range is numpy's stable sort of the
    assignments routed to held experts, i.e. exactly the rows [offsets[b], offsets[b+n]) of the
    dispatch over all experts; the other assignments get inv_perm = -1."""
    rng = np.random.default_rng(13)
    T, E, k = 300, 128, 8
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, st, ip = O.permute(ids, E, held=(b, n))
    flat = ids.ravel()
    held = (flat >= b) & (flat < b + n)
    want_counts = np.bincount(flat[held], minlength=E)
    assert np.array_equal(counts, want_counts)
    assert offsets[0] == 0 and np.array_equal(offsets[1:], np.cumsum(want_counts))
    order = np.argsort(np.where(held, flat, E), kind="stable")[: held.sum()]
    assert np.array_equal(st[: held.sum()], order // k)
    assert np.all(ip[~held] == -1)
    assert np.array_equal(ip[order], np.arange(held.sum()))
    # the same rows as the full dispatch's slice
    _, off_all, st_all, ip_all = O.permute(ids, E)
    lo, hi = off_all[b], off_all[b + n]
    assert np.array_equal(st[: held.sum()], st_all[lo:hi])
    assert np.array_equal(ip[held], ip_all[held] - lo)


def _share(inp, b, n):
    """The inputs a rank holding experts [b, b+n) sees: every token, its experts' weights."""
    out = dict(inp)
    for key in ("w13", "w2", "w13_scale", "w2_scale", "w13_gscale", "w2_gscale"):
        if inp.get(key) is not None:
            out[key] = np.ascontiguousarray(inp[key][b:b + n])
    return out


@pytest.mark.parametrize("wdt", ["f32", "bf16", "nvfp4", "mxfp8", "mxfp4"])
def test_partial_outputs_over_an_expert_partition_sum_to_the_layer(wdt):
    wl, inp = _tiny(wdt=wdt, T=24, H=64, E=8, k=3, F=64 if wdt.startswith("mx") else 48)
    full = O.forward(inp, wl.top_k, wl.wdt, wl.ffn)
    total = np.zeros_like(full["y"])
    for b, n in ((0, 3), (3, 2), (5, 3)):
        part = O.forward(_share(inp, b, n), wl.top_k, wl.wdt, wl.ffn, held=(b, n))
        assert np.array_equal(part["topk_ids"], full["topk_ids"])
        # a token's partial output is the weighted sum over its held experts only
        y_bf, _, _ = BF.layer(inp, full["logits"], wl.top_k, wdt, keep=lambda e: b <= e < b + n)
        np.testing.assert_allclose(part["y"], y_bf, rtol=1e-10, atol=1e-13)
        total += part["y"]
    np.testing.assert_allclose(total, full["y"], rtol=1e-12, atol=1e-14)


def test_held_range_of_all_experts_is_the_single_gpu_layer():
    wl, inp = _tiny(T=16, E=8, k=2)
    a = O.forward(inp, 2, wl.wdt, wl.ffn)
    b = O.forward(inp, 2, wl.wdt, wl.ffn, held=(0, 8))
    for key in ("counts", "offsets", "sorted_token", "inv_perm", "y"):
        assert np.array_equal(a[key], b[key]), key


def test_token_with_no_held_expert_gets_zero():
    wl, inp = _tiny(T=40, E=8, k=1)
    e = int(O.route(inp, 1)["topk_ids"][0, 0])  # an expert that some token picks
    r = O.forward(_share(inp, e, 1), 1, wl.wdt, wl.ffn, held=(e, 1))
    none = r["topk_ids"][:, 0] != e
    assert none.any() and (~none).any()
    assert np.all(r["y"][none] == 0.0) and np.all(np.abs(r["y"][~none]).max(1) > 0)


def test_pages_load_example_tokens_per_expert():
    g = json.load(open(os.path.join(GOLD, "pages_values.json")))["prefill_tokens_per_expert"]
    rng = np.random.default_rng(11)
    T, E, k = g["tokens"], g["experts"], g["top_k"]
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, _, _ = O.permute(ids, E)
    assert offsets[-1] == T * k and counts.mean() == g["per_expert"]


# ---------------------------------------------------------------------------------------
# expert FFN and the whole layer
# ---------------------------------------------------------------------------------------

def _tiny(wdt="f32", T=12, H=64, E=4, k=2, F=32, seed=0, act=None):
    act = act or ("f32" if wdt == "f32" else "bf16")
    wl = synth.Workload("t", T, H, E, k, F, act, wdt, seed, "normal")
    return wl, synth.generate(wl)


def test_identical_experts_equal_dense_swiglu_mlp():
    wl, inp = _tiny(E=6, k=3, T=20)
    inp["w13"][:] = inp["w13"][0]
    inp["w2"][:] = inp["w2"][0]
    r = O.forward(inp, wl.top_k, wl.wdt, wl.ffn)
    x = inp["x"].astype(np.float64)
    w13 = inp["w13"][0].astype(np.float64)
    w2 = inp["w2"][0].astype(np.float64)
    g, u = x @ w13[: wl.ffn].T, x @ w13[wl.ffn:].T
    dense = (g * scipy.special.expit(g) * u) @ w2.T
    np.testing.assert_allclose(r["y"], dense, rtol=1e-10, atol=1e-14)


def test_single_expert_top1_is_dense_mlp():
    wl, inp = _tiny(E=1, k=1, T=7)
    r = O.forward(inp, 1, wl.wdt, wl.ffn)
    x = inp["x"].astype(np.float64)
    w13, w2 = inp["w13"][0].astype(np.float64), inp["w2"][0].astype(np.float64)
    g, u = x @ w13[: wl.ffn].T, x @ w13[wl.ffn:].T
    np.testing.assert_allclose(r["y"], (g / (1 + np.exp(-g)) * u) @ w2.T, rtol=1e-12, atol=1e-15)
    assert np.all(r["topk_w"] == 1.0)


def test_zero_tokens_give_zero_output():
    wl, inp = _tiny()
    inp["x"][:] = 0
    r = O.forward(inp, wl.top_k, wl.wdt, wl.ffn)
    assert np.all(r["y"] == 0.0)
    assert np.array_equal(r["logits"], np.broadcast_to(inp["bias"], r["logits"].shape))


def test_top1_combine_returns_the_expert_row():
    wl, inp = _tiny(k=1)
    r = O.forward(inp, 1, wl.wdt, wl.ffn)
    rows = O.expert_rows(inp, wl.wdt, wl.ffn, np.arange(wl.tokens), r["topk_ids"][:, 0])
    assert np.array_equal(r["y"], rows)


@pytest.mark.parametrize("wdt", ["f32", "bf16", "nvfp4", "mxfp8", "mxfp4"])
def test_layer_matches_per_token_bruteforce(wdt):
    wl, inp = _tiny(wdt=wdt, T=24, H=64, E=8, k=3, F=64 if wdt.startswith("mx") else 48)
    r = O.forward(inp, wl.top_k, wl.wdt, wl.ffn)
    y, ids, w = BF.layer(inp, r["logits"], wl.top_k, wdt)
    assert np.array_equal(r["topk_ids"], ids)
    np.testing.assert_allclose(r["topk_w"], w, rtol=1e-12)
    np.testing.assert_allclose(r["y"], y, rtol=1e-10, atol=1e-13)


def test_layer_full_softmax_weights_option():
    wl, inp = _tiny(T=10, E=8, k=3)
    r = O.forward(inp, 3, wl.wdt, wl.ffn, renormalize=False)
    y, ids, w = BF.layer(inp, r["logits"], 3, wl.wdt, renormalize=False)
    np.testing.assert_allclose(r["y"], y, rtol=1e-10, atol=1e-13)
    assert np.all(r["topk_w"].sum(1) < 1)


def test_token_sample_equals_full_run():
    wl, inp = _tiny(T=30, E=8, k=3)
    full = O.forward(inp, 3, wl.wdt, wl.ffn)
    toks = np.array([29, 0, 7, 7, 13])
    part = O.forward(inp, 3, wl.wdt, wl.ffn, tokens=toks)
    assert np.array_equal(part["y"], full["y"][toks])


def test_nvfp4_quantiser_round_trips_within_fp4_error():
    w = np.random.default_rng(12).standard_normal((8, 64)).astype(np.float32) * 0.02
    packed, sc, g = synth.quantize_nvfp4(w)
    codes = np.stack([packed & 15, packed >> 4], -1).reshape(8, 64)
    deq = O.decode_e2m1(codes) * np.repeat(O.decode_e4m3(sc), 16, 1) * g
    bmax = np.repeat(np.abs(w).reshape(8, 4, 16).max(2), 16, 1)
    assert np.all(np.abs(deq - w) <= 0.25 * bmax * 1.07 + 1e-12)


def test_generator_is_deterministic_and_expert_subsets_agree():
    wl = synth.Workload("t", 4, 64, 6, 2, 32, "bf16", "nvfp4", 77, "normal")
    a = synth.generate(wl)
    b = synth.generate(wl, experts=[5, 2])
    assert synth.digest(a) == synth.digest(synth.generate(wl))
    for key in ("w13", "w2", "w13_scale", "w2_scale", "w13_gscale", "w2_gscale"):
        assert np.array_equal(b[key], a[key][[5, 2]])


@pytest.mark.slow
def test_hot_set_receives_half_of_the_assignments():
    wl = synth.WORKLOADS["nvfp4_prefill"]
    inp = synth.generate(wl, with_experts=False)
    r = O.route(inp, wl.top_k)
    share = np.isin(r["topk_ids"], synth.hot_set(wl)).mean()
    assert abs(share - synth.HOT_SHARE_TARGET) <= 0.005
    assert len(synth.hot_set(wl)) == 26


def test_p99_error_metric_on_known_values():
    """The per-element error figure the GPU tests report: 99th percentile of
    |got - ref| / (|ref| + 1e-3 rms(ref)).  On 1000 elements of value 1 with the first 6 off by
    0.25 and the last 5 off by 0.5, the 99th percentile falls between the two error levels."""
    import sys, os
    sys.path.insert(0, os.path.dirname(__file__))
    from gpu_checks import p99_err
    ref = np.ones(1000)
    got = ref.copy()
    got[-5:] += 0.5
    got[:6] += 0.25
    rms = 1.0
    e = p99_err(got, ref)
    # sorted errors: 989 zeros, 6 at 0.25/(1+1e-3), 5 at 0.5/(1+1e-3); rank 989.01 of 999
    assert 0.25 / (1 + 1e-3 * rms) - 1e-12 <= e <= 0.5 / (1 + 1e-3 * rms) + 1e-12
    assert p99_err(ref, ref) == 0.0
