"""Pins for the router steps (S1-S2): brute-force selection, closed-form
weights, the bias invariant, ties, NaN ordering, the k bound."""
import itertools
import math

import numpy as np
import pytest

from oracle import moe_oracle as mo


def _beats(a, sa, b, sb):
    """Brute-force ranking rule written from scratch: a larger biased score
    wins; a number beats NaN; on equal scores (or both NaN) the lower id."""
    na, nb = math.isnan(sa), math.isnan(sb)
    if na and nb:
        return a < b
    if na != nb:
        return nb
    return sa > sb or (sa == sb and a < b)


def brute_force_set(sb_row, k):
    """The unique k-subset whose every member ranks before every
    non-member (checked over all C(E,k) subsets)."""
    E = len(sb_row)
    winners = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(_beats(a, float(sb_row[a]), b, float(sb_row[b])) for a in S for b in rest):
            winners.append(S)
    assert len(winners) == 1, winners
    return list(winners[0])


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_with_ties_and_nans(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 11))
    k = int(rng.integers(1, E + 1))
    T = 40
    # a coarse grid of logits and biases makes exact ties frequent
    logits = rng.integers(-3, 4, size=(T, E)).astype(np.float32) * np.float32(0.5)
    bias = (rng.integers(-2, 3, size=E) * 0.125).astype(np.float32)
    nan_mask = rng.random((T, E)) < 0.08
    logits[nan_mask] = np.nan
    r = mo.topk_route(logits, bias, k, rsf=1.5)
    for t in range(T):
        assert list(r["ids"][t]) == brute_force_set(r["s_biased"][t], k), t


def test_ids_ascending_and_distinct():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((200, 32)).astype(np.float32)
    r = mo.topk_route(logits, rng.uniform(-.1, .1, 32).astype(np.float32), 8, 1.0)
    assert np.all(np.diff(r["ids"], axis=1) > 0)


def test_weights_closed_form_and_sigmoid_zero():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((50, 12)).astype(np.float32) * 3
    logits[:, 0] = 0.0
    bias = np.full(12, 0.0, np.float32)
    bias[0] = 10.0            # force expert 0 into every selection
    rsf = 2.5
    r = mo.topk_route(logits, bias, 4, rsf)
    assert np.all(r["ids"][:, 0] == 0)
    # sigmoid(0) = 1/2 exactly -> w = rsf/2 exactly
    assert np.all(r["w"][:, 0] == np.float32(1.25))
    for t in range(50):
        for j, e in enumerate(r["ids"][t]):
            sig = 1.0 / (1.0 + math.exp(-float(logits[t, e])))
            expect = np.float32(np.float32(rsf) * np.float32(sig))
            assert r["w"][t, j] == expect
    assert np.all(r["w"] > 0) and np.all(r["w"] <= rsf)


@pytest.mark.parametrize("seed", range(3))
def test_bias_never_changes_an_emitted_weight(seed):
    rng = np.random.default_rng(seed)
    T, E, k = 300, 16, 4
    logits = rng.standard_normal((T, E)).astype(np.float32)
    b1 = rng.uniform(-.5, .5, E).astype(np.float32)
    b2 = rng.uniform(-.5, .5, E).astype(np.float32)
    r1 = mo.topk_route(logits, b1, k, 1.7)
    r2 = mo.topk_route(logits, b2, k, 1.7)
    changed = 0
    for t in range(T):
        d1 = dict(zip(r1["ids"][t], r1["w"][t]))
        d2 = dict(zip(r2["ids"][t], r2["w"][t]))
        changed += set(d1) != set(d2)
        for e in set(d1) & set(d2):
            assert d1[e].tobytes() == d2[e].tobytes()
    assert changed > 0      # the biases did steer some selections


def test_router_logits_are_fp32_of_exact_products():
    """x bf16 widened exactly, fp32 weights: the logit is the fp32 rounding
    of the exact dot product (math.fsum)."""
    rng = np.random.default_rng(3)
    import moe_inputs
    x = moe_inputs.f32_to_bf16_bits(rng.standard_normal((7, 33)).astype(np.float32))
    wr = (rng.standard_normal((5, 33)) * 0.02).astype(np.float32)
    l = mo.router_logits(x, wr)
    xf = moe_inputs.bf16_bits_to_f32(x).astype(np.float64)
    for t in range(7):
        for e in range(5):
            exact = math.fsum(float(a) * float(b) for a, b in zip(xf[t], wr[e].astype(np.float64)))
            assert l[t, e] == np.float32(exact)


def test_full_expert_count_selection_is_row_independent():
    """Routing a token alone or inside a batch, in any order, gives the
    same ids (every rank ranks all experts on its own)."""
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((64, 20)).astype(np.float32)
    b = rng.uniform(-.1, .1, 20).astype(np.float32)
    full = mo.topk_route(logits, b, 6, 1.0)["ids"]
    perm = rng.permutation(64)
    shuffled = mo.topk_route(logits[perm], b, 6, 1.0)["ids"]
    np.testing.assert_array_equal(shuffled, full[perm])
    for t in (0, 17, 63):
        np.testing.assert_array_equal(mo.topk_route(logits[t:t + 1], b, 6, 1.0)["ids"][0], full[t])


def test_k_bounds():
    l = np.zeros((2, 20), np.float32)
    with pytest.raises(ValueError):
        mo.topk_route(l, None, 0, 1.0)
    with pytest.raises(ValueError):
        mo.topk_route(l, None, 17, 1.0)
    with pytest.raises(ValueError):
        mo.topk_route(l[:, :4], None, 5, 1.0)
    r = mo.topk_route(np.zeros((2, 16), np.float32), None, 16, 1.0)
    assert list(r["ids"][0]) == list(range(16))
    assert np.all(np.isinf(r["gap"]))


def test_gap_is_kth_minus_next():
    s = np.array([[0.9, 0.1, 0.5, 0.5000001, 0.2]], np.float32)
    logits = np.log(s / (1 - s)).astype(np.float32)
    r = mo.topk_route(logits, None, 2, 1.0)
    sb = np.sort(r["s_biased"][0].astype(np.float64))[::-1]
    assert r["gap"][0] == pytest.approx(sb[1] - sb[2])
    assert r["gap"][0] < 1e-5
