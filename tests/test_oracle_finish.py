"""Pins of the oracle's finish step S8 (the residual add after the layer
output, "bridge.models.beam.modeling_beam": scaled_residual_add and _beam_bda;
"core.models.hybrid.shortcut_block": ShortcutMoEBlock._postprocess) and of
the post-norm on a plain layer (Beam's sandwich norm on the MLP output).

The pages define the add as output * coefs[0] + residual * coefs[1] in the
residual's dtype; the pins hold it to hand-worked bf16 values, to PyTorch's
own bf16 tensor arithmetic (the pages' formula run literally), and to the
identities it must satisfy."""
import numpy as np
import torch

import moe_inputs
from oracle import moe_oracle as mo


def _b(v):
    return moe_inputs.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _v(bits):
    return moe_inputs.bf16_bits_to_f32(bits).astype(np.float64)


def test_finish_hand_values():
    # c0 = c1 = 1: bf16(o + r).  1 + 2^-8 lies halfway between the bf16
    # neighbours 1 and 1 + 2^-7 -> ties to even -> 1;  1 + 3*2^-9 is past
    # the midpoint -> 1 + 2^-7;  1 + 1 = 2 exactly.
    out = mo.finish(_b([1.0, 1.0, 1.0]), _b([2.0 ** -8, 3 * 2.0 ** -9, 1.0]))
    assert _v(out).tolist() == [1.0, 1.0078125, 2.0]
    # depth-scaled (0.6, 0.8), o = r = 1: bf16(0.6) = 77/128 (0.6015625:
    # 0.2 * 128 = 25.6 -> 26 over 2^-1), bf16(0.8) = 205/256 (0.80078125);
    # their sum 1.40234375 = 1 + 51.5/128 is a tie -> 52 -> 1.40625.  A
    # single rounding of 0.6 + 0.8 would give 1 + 51/128 = 1.3984375.
    out = mo.finish(_b([1.0]), _b([1.0]), 0.6, 0.8)
    assert _v(out).tolist() == [1.40625]


def test_finish_is_torch_bf16_arithmetic():
    rng = np.random.default_rng(11)
    o = _b(rng.standard_normal(20000))
    r = _b(rng.standard_normal(20000) * 4)
    ot = torch.from_numpy(o.view(np.int16)).view(torch.bfloat16)
    rt = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
    for c0, c1 in [(1.0, 1.0), (0.6, 0.8), (2 ** -0.5, 2 ** -0.5), (0.25, 0.9682458365518543)]:
        ref = (ot * c0 + rt * c1).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(mo.finish(o, r, c0, c1), ref), (c0, c1)


def test_finish_identities():
    rng = np.random.default_rng(12)
    o = _b(rng.standard_normal(4096))
    r = _b(rng.standard_normal(4096))
    assert np.array_equal(mo.finish(o, r, 1.0, 0.0), o)           # no residual term
    assert np.array_equal(mo.finish(o, r, 0.6, 0.8), mo.finish(r, o, 0.8, 0.6))  # commutes
    # powers of two scale exactly: bf16(o / 2 + r / 2) == bf16 of the exact sum / 2
    half = mo.finish(o, r, 0.5, 0.5)
    full = mo.finish(o, r, 1.0, 1.0)
    assert np.array_equal(_v(half) * 2, _v(full))


def _small():
    wl = moe_inputs.Workload("fin", T=12, H=128, E=6, k=2, I=64, I_s=64)
    return wl, moe_inputs.generate(wl, 3)


def test_plain_post_norm_wiring():
    wl, inp = _small()
    inp["gamma_post"] = (1 + 0.1 * np.random.default_rng(4).uniform(-1, 1, wl.H)).astype(np.float32)
    plain = mo.forward(inp, k=wl.k, rsf=wl.rsf, limit=wl.limit)
    normed = mo.forward(inp, k=wl.k, rsf=wl.rsf, limit=wl.limit, post_norm=True, eps=1e-6)
    assert np.array_equal(normed["z"], plain["z"])
    # each row of the output over its gains has RMS sqrt(ms / (ms + eps)),
    # ms the row's mean square of z (bf16 rounding aside)
    v = _v(normed["out"]) / inp["gamma_post"].astype(np.float64)
    ms = np.mean(plain["z"] ** 2, axis=1)
    assert np.allclose(np.sqrt(np.mean(v * v, axis=1)), np.sqrt(ms / (ms + 1e-6)), rtol=5e-3)
    assert np.array_equal(normed["out"],
                          mo.bf16_round(mo.rmsnorm_f64(plain["z"], inp["gamma_post"], 1e-6)))


def test_forward_with_residual():
    wl, inp = _small()
    res = _b(np.random.default_rng(5).standard_normal((wl.T, wl.H)))
    base = mo.forward(inp, k=wl.k, rsf=wl.rsf, limit=wl.limit)
    fin = mo.forward(inp, k=wl.k, rsf=wl.rsf, limit=wl.limit, residual=res,
                     out_scale=0.6, residual_scale=0.8)
    assert np.array_equal(fin["out_layer"], base["out"])
    assert np.array_equal(fin["out"], mo.finish(base["out"], res, 0.6, 0.8))
