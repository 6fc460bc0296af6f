"""Planted mistakes (in the oracle, on the CPU): each plausible error in the
layer's arithmetic must make at least one pin fail.  This shows the pins
are sharp enough to trust the oracle."""
import numpy as np
import pytest

from oracle import moe_oracle as mo
from tests.helpers import load_hand_example


def _hand_matches():
    inp, p, exp = load_hand_example()
    res = mo.forward(inp, k=p["k"], rsf=p["rsf"], limit=p["limit"])
    ok = (np.array_equal(res["ids"], exp["ids"])
          and np.allclose(res["w"], exp["w"], rtol=1e-8)
          and np.allclose(res["z"], exp["z"], rtol=1e-8, atol=1e-9)
          and np.array_equal(mo.bf16_to_f64(res["out"]), np.asarray(exp["out"], np.float64)))
    return ok


def test_unmutated_oracle_matches():
    assert _hand_matches()


def _symmetric_clamp(a, w_gate_up, w_down, limit, round_h=True, h_given=None):
    I = w_gate_up.shape[0] // 2
    g = a @ mo.bf16_to_f64(w_gate_up[:I]).T
    u = a @ mo.bf16_to_f64(w_gate_up[I:]).T
    gc = np.clip(g, -limit, limit)
    h = gc / (1 + np.exp(-gc)) * np.clip(u, -limit, limit)
    if round_h:
        h = mo.bf16_to_f64(mo.bf16_round(h))
    return h, h @ mo.bf16_to_f64(w_down).T


def _swapped_gate_up(a, w_gate_up, w_down, limit, round_h=True, h_given=None):
    I = w_gate_up.shape[0] // 2
    sw = np.concatenate([w_gate_up[I:], w_gate_up[:I]])
    return _real_ffn(a, sw, w_down, limit, round_h, h_given)


_real_ffn = mo.swiglu_ffn
_real_route = mo.topk_route
_real_combine = mo.combine


def _biased_weights(logits, corr_bias, k, rsf):
    r = _real_route(logits, corr_bias, k, rsf)
    r["w"] = (np.float32(rsf) * np.take_along_axis(r["s_biased"], r["ids"], 1)).astype(np.float32)
    return r


def _renormalised(logits, corr_bias, k, rsf):
    r = _real_route(logits, corr_bias, k, rsf)
    w = np.take_along_axis(r["s"], r["ids"], 1).astype(np.float64)
    r["w"] = (rsf * w / w.sum(1, keepdims=True)).astype(np.float32)
    return r


def _bias_on_logit(logits, corr_bias, k, rsf):
    shifted = (logits + corr_bias[None, :]).astype(np.float32)
    r = _real_route(shifted, None, k, rsf)
    r["w"] = (np.float32(rsf) * np.take_along_axis(mo.sigmoid_f32(logits), r["ids"], 1)).astype(np.float32)
    return r


def _ties_to_higher_id(logits, corr_bias, k, rsf):
    E = logits.shape[1]
    r = _real_route(logits[:, ::-1].copy(), corr_bias[::-1].copy(), k, rsf)
    ids = np.sort(E - 1 - r["ids"], axis=1).astype(np.int32)
    r["ids"] = ids
    r["w"] = (np.float32(rsf) * np.take_along_axis(mo.sigmoid_f32(logits), ids, 1)).astype(np.float32)
    return r


def _shared_scaled(y_perm, w, inv_pos, ys):
    return _real_combine(y_perm, w, inv_pos, None if ys is None else 2.5 * ys)


@pytest.mark.parametrize("name,attr,fake", [
    ("symmetric clamp", "swiglu_ffn", _symmetric_clamp),
    ("gate/up swapped", "swiglu_ffn", _swapped_gate_up),
    ("weights carry the bias", "topk_route", _biased_weights),
    ("weights renormalised", "topk_route", _renormalised),
    ("bias on the logit", "topk_route", _bias_on_logit),
    ("ties to the higher id", "topk_route", _ties_to_higher_id),
    ("shared expert scaled", "combine", _shared_scaled),
])
def test_planted_mistake_is_caught(monkeypatch, name, attr, fake):
    monkeypatch.setattr(mo, attr, fake)
    assert not _hand_matches(), name


# Planted mistakes in the finish step S8: each must fail a pin of
# test_oracle_finish (run here against the mutated function).
_real_finish = mo.finish


def _finish_one_rounding(o, r, c0=1.0, c1=1.0):
    v = mo.bf16_to_f64(o) * c0 + mo.bf16_to_f64(r) * c1
    return mo.bf16_round(v)


def _finish_scales_swapped(o, r, c0=1.0, c1=1.0):
    return _real_finish(o, r, c1, c0)


@pytest.mark.parametrize("name,fake", [
    ("finish rounded once", _finish_one_rounding),
    ("finish scales swapped", _finish_scales_swapped),
])
def test_planted_finish_mistake_is_caught(monkeypatch, name, fake):
    from tests import test_oracle_finish as pins
    monkeypatch.setattr(mo, "finish", fake)
    failed = 0
    for pin in (pins.test_finish_hand_values, pins.test_finish_is_torch_bf16_arithmetic,
                pins.test_finish_identities):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, name


# Planted mistakes in the ScMoE pre-norm gain: each must fail a pin of the
# pre-norm (the hand-worked gain, the per-channel scaling of the routed
# input, the gained routing).
_real_rmsnorm_bf16 = mo.rmsnorm_bf16


def _gain_ignored(x_bits, gamma, eps):
    return _real_rmsnorm_bf16(x_bits, None, eps)


def _gain_inverted(x_bits, gamma, eps):
    inv = None if gamma is None else (1.0 / np.asarray(gamma, np.float64)).astype(np.float32)
    return _real_rmsnorm_bf16(x_bits, inv, eps)


_real_forward = mo.forward


def _post_gain_used_before_routing(inp, **kw):
    # the forward hands the post-norm gain to the pre-norm
    return _real_forward(dict(inp, gamma_pre=inp.get("gamma_post")), **kw)


@pytest.mark.parametrize("name,fake", [
    ("pre-norm gain ignored", _gain_ignored),
    ("pre-norm gain inverted", _gain_inverted),
])
def test_planted_pre_gain_mistake_is_caught(monkeypatch, name, fake):
    from tests import test_oracle_layer as pins
    monkeypatch.setattr(mo, "rmsnorm_bf16", fake)
    failed = 0
    for pin in (pins.test_rmsnorm_gain_closed_form,
                pins.test_scmoe_pre_gain_scales_routed_input_per_channel,
                pins.test_scmoe_routes_the_gained_input):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 2, name


def test_planted_gain_swap_is_caught(monkeypatch):
    from tests import test_oracle_layer as pins
    monkeypatch.setattr(mo, "forward", _post_gain_used_before_routing)
    with pytest.raises(AssertionError):
        pins.test_scmoe_pre_gain_scales_routed_input_per_channel()


# Planted mistakes in the W4A16 dequantisation: each must fail a W4 pin.
_real_e4m3 = mo.e4m3_to_f64
_real_dequant_w4 = mo.dequant_w4


def _e4m3_bias_8(codes):
    return _real_e4m3(codes) / 2.0


def _e4m3_no_subnormals(codes):
    b = np.asarray(codes, np.uint8)
    v = _real_e4m3(b)
    return np.where(((b >> 3) & 0xF) == 0, np.sign(v) * (1 + (b & 7) / 8.0) * 2.0 ** -7, v)


def _tensor_scale_ignored(q, scale_codes, tensor_scale=1.0):
    return _real_dequant_w4(q, scale_codes, 1.0)


@pytest.mark.parametrize("name,attr,fake", [
    ("E4M3 exponent bias 8", "e4m3_to_f64", _e4m3_bias_8),
    ("E4M3 subnormals read as normals", "e4m3_to_f64", _e4m3_no_subnormals),
    ("tensor scale ignored", "dequant_w4", _tensor_scale_ignored),
])
def test_planted_w4_mistake_is_caught(monkeypatch, name, attr, fake):
    from tests import test_oracle_w4 as pins
    monkeypatch.setattr(mo, attr, fake)
    failed = 0
    for pin in (pins.test_e4m3_hand_values, pins.test_e4m3_every_byte_matches_torch,
                pins.test_dequant_hand_example, pins.test_dequant_matches_packer_and_scales):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, name
