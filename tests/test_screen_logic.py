"""CPU check of the screening rule the large-batch router uses (route.hip): given approximate
logits m with |l - m| <= beta for the canonical logits l, let tau be the k-th largest m - beta;
experts with m + beta < tau cannot be among the k largest l (ties to the lower index), so keeping
the canonical logits of the others and -inf elsewhere selects the same ids with the same weights.

Here the rule runs in numpy on the oracle's canonical logits with adversarial perturbations
inside the bound (selected experts pushed down by beta, the others pushed up, random signs, exact
ties from duplicated router rows and zero tokens); the oracle's selection on the screened logits
must equal its selection on the full logits.  The bound itself (that the matrix-core logits lie
within beta) is a property of the GPU path, checked there bit for bit against the full router."""
import numpy as np
import pytest

from mixture_experts_layer_softmax_amd import synth
from oracle import oracle as O


def screen(l, m, beta, k):
    lo = m - beta
    tau = -np.sort(-lo, axis=1)[:, k - 1]
    cand = m + beta >= tau[:, None]
    out = np.where(cand, l, -np.inf).astype(np.float32)
    return out, cand


def canonical_logits(T, H, E, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[: T // 8] = 0.0                                    # logits = bias: ties everywhere
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    wr[1::5] = wr[0::5][: len(wr[1::5])]                 # duplicated experts: exact ties
    bias = rng.choice(np.array([0.0, 0.25], np.float32), size=E)
    return O.router_logits(synth.to_bf16_bits(x), synth.to_bf16_bits(wr), bias)


@pytest.mark.parametrize("E,k,beta", [(32, 4, 0.05), (128, 8, 0.02), (256, 8, 0.3), (64, 16, 0.01),
                                      (16, 16, 0.1)])
@pytest.mark.parametrize("mode", ["adversarial", "random", "exact"])
def test_screened_selection_equals_full_selection(E, k, beta, mode):
    T, H = 96, 256
    l = canonical_logits(T, H, E, seed=E * 7 + k)
    ids_ref, w_ref = O.select(l, k)
    rng = np.random.default_rng(3)
    # perturbations strictly inside the bound: at exactly +-beta the float rounding of m +- beta
    # decides the boundary, which the kernel's bound covers with a |m| 2^-21 margin
    d = beta * (1 - 2.0 ** -10)
    if mode == "adversarial":  # the selected experts look worse, the others better, by the bound
        sel = np.zeros_like(l, dtype=bool)
        np.put_along_axis(sel, ids_ref.astype(np.int64), True, axis=1)
        delta = np.where(sel, -d, d)
    elif mode == "random":
        delta = rng.uniform(-d, d, size=l.shape)
    else:
        delta = np.zeros_like(l)
    m = l.astype(np.float64) + delta
    screened, cand = screen(l, m, np.full_like(m, beta), k)
    assert np.all(cand.sum(axis=1) >= k)
    ids, w = O.select(screened, k)
    assert np.array_equal(ids, ids_ref)
    assert np.array_equal(w, w_ref)


def test_a_bound_too_small_can_change_the_selection():
    """The rule needs |l - m| <= beta: with perturbations of twice the assumed bound, the
    adversarial case drops a selected expert (so the checks above are not vacuous)."""
    T, H, E, k, beta = 96, 256, 128, 8, 0.02
    l = canonical_logits(T, H, E, seed=11)
    ids_ref, _ = O.select(l, k)
    sel = np.zeros_like(l, dtype=bool)
    np.put_along_axis(sel, ids_ref.astype(np.int64), True, axis=1)
    m = l.astype(np.float64) + np.where(sel, -2 * beta, 2 * beta)
    screened, _ = screen(l, m, np.full_like(m, beta), k)
    ids, _ = O.select(screened, k)
    assert not np.array_equal(ids, ids_ref)
