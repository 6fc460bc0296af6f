"""Pins for the permutation (S3): invariants, a library routine, and the
loop rendering."""
import numpy as np
import pytest

from oracle import moe_oracle as mo
from oracle import loops


def _random_ids(rng, T, E, k):
    return np.stack([np.sort(rng.choice(E, size=k, replace=False)) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 3, 2), (64, 8, 2), (300, 64, 8), (257, 256, 16)])
def test_permute_invariants(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    ids = _random_ids(rng, T, E, k)
    p = mo.permute(ids, E)
    off, st, inv = p["offsets"], p["sorted_token"], p["inv_pos"]
    assert off[0] == 0 and off[E] == T * k
    assert np.all(np.diff(off) >= 0)
    assert np.array_equal(np.diff(off), np.bincount(ids.ravel(), minlength=E))
    # inv_pos is a bijection onto 0..T*k-1
    assert np.array_equal(np.sort(inv), np.arange(T * k))
    flat = ids.ravel()
    for e in range(E):
        seg = slice(off[e], off[e + 1])
        toks = st[seg]
        assert np.all(np.diff(toks) > 0)                   # ascending tokens
    # each pair lands in its expert's segment, on a row holding its token
    for pair in range(T * k):
        row = inv[pair]
        e = flat[pair]
        assert off[e] <= row < off[e + 1]
        assert st[row] == pair // k


def test_permute_equals_stable_library_sort():
    rng = np.random.default_rng(9)
    ids = _random_ids(rng, 500, 37, 5)
    p = mo.permute(ids, 37)
    # an independent construction: Python's sorted (stable) on (id, pair)
    pairs = sorted(range(ids.size), key=lambda q: (int(ids.ravel()[q]), q))
    assert list(p["sorted_token"]) == [q // 5 for q in pairs]


def test_permute_equals_loop_rendering():
    rng = np.random.default_rng(10)
    ids = _random_ids(rng, 40, 9, 3)
    p = mo.permute(ids, 9)
    off, st, inv = loops.permute_loops(ids.tolist(), 9)
    assert list(p["offsets"]) == off
    assert list(p["sorted_token"]) == st
    assert list(p["inv_pos"]) == inv


def test_permute_empty_experts_and_empty_batch():
    ids = np.array([[0, 3], [0, 3]], np.int32)
    p = mo.permute(ids, 6)
    assert list(p["offsets"]) == [0, 2, 2, 2, 4, 4, 4]
    p0 = mo.permute(np.zeros((0, 4), np.int32), 6)
    assert list(p0["offsets"]) == [0] * 7
    assert p0["sorted_token"].size == 0
