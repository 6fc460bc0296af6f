"""Pin: the oracle reproduces the hand-worked example value by value.

The example (tests/golden/hand_example.json) covers a selection changed
by the bias alone, an exact tie, an expert never chosen, all four clamp
branches, the unscaled shared expert and the bf16 rounding points.
"""
import numpy as np
import pytest

from oracle import moe_oracle as mo
from tests.helpers import load_hand_example


@pytest.fixture(scope="module")
def hand():
    inp, p, exp = load_hand_example()
    res = mo.forward(inp, k=p["k"], rsf=p["rsf"], limit=p["limit"])
    return inp, p, exp, res


def test_logits(hand):
    _, _, exp, res = hand
    np.testing.assert_array_equal(res["logits"], np.asarray(exp["logits"], np.float32))


def test_ids_and_weights(hand):
    _, _, exp, res = hand
    np.testing.assert_array_equal(res["ids"], exp["ids"])
    np.testing.assert_allclose(res["w"], exp["w"], rtol=1e-8, atol=0)
    # sigmoid(0) = 1/2 exactly, so rsf * 1/2 is exact
    assert res["w"][0, 0] == np.float32(1.25)
    assert res["w"][3, 1] == np.float32(1.25)


def test_permutation(hand):
    _, _, exp, res = hand
    np.testing.assert_array_equal(res["offsets"], exp["offsets"])
    np.testing.assert_array_equal(res["sorted_token"], exp["sorted_token"])
    np.testing.assert_array_equal(res["inv_pos"], exp["inv_pos"])


def test_h_values_and_clamp_branches(hand):
    _, p, exp, res = hand
    ids = res["ids"]
    k = p["k"]
    hb = exp["h_bf16"]
    for t in range(p["T"]):
        for j in range(k):
            e = int(ids[t, j])
            row = res["inv_pos"][t * k + j]
            assert res["h_perm"][row, 0] == hb[f"t{t}e{e}"], (t, e)
    np.testing.assert_array_equal(res["hs"][:, 0], exp["hs_bf16"])


def test_h_exact_without_rounding(hand):
    inp, p, exp, _ = hand
    res = mo.forward(inp, k=p["k"], rsf=p["rsf"], limit=p["limit"], round_h=False)
    for key, v in exp["h_exact"].items():
        t, e = int(key[1]), int(key[3])
        j = list(res["ids"][t]).index(e)
        row = res["inv_pos"][t * p["k"] + j]
        assert res["h_perm"][row, 0] == pytest.approx(v, rel=1e-8)
    np.testing.assert_allclose(res["z"], exp["z_without_h_rounding"], rtol=1e-8, atol=1e-9)


def test_combine_and_output(hand):
    _, _, exp, res = hand
    np.testing.assert_allclose(res["z"], exp["z"], rtol=1e-8, atol=1e-9)
    out = mo.bf16_to_f64(res["out"])
    np.testing.assert_array_equal(out, np.asarray(exp["out"], np.float64))


def test_bias_only_steers_selection(hand):
    inp, p, exp, res = hand
    inp0 = dict(inp, corr_bias=np.zeros(p["E"], np.float32))
    res0 = mo.forward(inp0, k=p["k"], rsf=p["rsf"], limit=p["limit"])
    np.testing.assert_array_equal(res0["ids"], exp["ids_bias_zero"])
    for t in range(p["T"]):
        for j, e in enumerate(res["ids"][t]):
            if e in res0["ids"][t]:
                j0 = list(res0["ids"][t]).index(e)
                assert res["w"][t, j].tobytes() == res0["w"][t, j0].tobytes()


def test_never_chosen_expert_is_never_computed(hand):
    """Expert 4 has huge weights; it is never selected, so any use of it
    would blow up the output."""
    _, _, _, res = hand
    assert res["offsets"][4] == res["offsets"][5]
    assert np.all(np.abs(res["z"]) < 100)
