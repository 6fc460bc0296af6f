"""Pins of the oracle's W4A16 expert weights (the format is this library's
reading; the pages name the W4A16 expert GEMM but not its layout):
hand-worked dequantisation, a nibble packer written out here, and the
special case where every dequantised weight is exact in bf16, in which the
W4A16 layer must equal the bf16 layer (pinned elsewhere) bit for bit."""
import numpy as np

import moe_inputs
from oracle import moe_oracle as mo


def _bf16(v):
    return moe_inputs.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _pack(codes):
    """codes: int array [R, K] of nibbles 0..15 -> bytes [R, K/2]: in each
    4-byte word of 8 columns, byte j holds column j (low nibble) and
    column j + 4 (high nibble) (written element by element)."""
    R, K = codes.shape
    out = np.zeros((R, K // 2), dtype=np.uint8)
    for r in range(R):
        for w in range(K // 8):
            for j in range(4):
                lo = int(codes[r, 8 * w + j])
                hi = int(codes[r, 8 * w + j + 4])
                out[r, 4 * w + j] = lo | (hi << 4)
    return out


def test_dequant_hand_example():
    # one row, K = 256: two groups of 128 columns
    q = np.full((1, 128), 0x88, dtype=np.uint8)   # nibble 8 everywhere -> 0
    q[0, 0] = 0x9F     # byte 0 of word 0: columns 0, 4: nibbles 15, 9 -> 7, 1
    q[0, 65] = 0x70    # byte 1 of word 16: columns 129, 133: nibbles 0, 7 -> -8, -1
    q[0, 127] = 0x0F   # byte 3 of word 31: columns 251, 255: nibbles 15, 0 -> 7, -8
    scale = _bf16([[0.5], [-2.0]])                 # [groups, rows]
    w = mo.dequant_w4(q, scale)
    assert w.shape == (1, 256)
    assert w[0, 0] == 3.5 and w[0, 4] == 0.5
    assert w[0, 129] == 16.0 and w[0, 133] == 2.0
    assert w[0, 251] == -14.0 and w[0, 255] == 16.0
    assert np.count_nonzero(w) == 6


def test_dequant_matches_packer_and_scales():
    rng = np.random.default_rng(5)
    R, K = 6, 384
    codes = rng.integers(0, 16, size=(R, K))
    scale = _bf16(rng.uniform(-1, 1, size=(K // 128, R)))
    w = mo.dequant_w4(_pack(codes), scale)
    s = moe_inputs.bf16_bits_to_f32(scale).astype(np.float64)
    for r in range(R):
        for c in range(0, K, 7):
            assert w[r, c] == (codes[r, c] - 8) * s[c // 128, r]


def _w4_exact_pair(seed):
    """A small workload in W4A16 form whose scales are powers of two (so
    every weight (u - 8) * s is exact in bf16), and the same layer with
    those weights stored as bf16."""
    wl = moe_inputs.Workload("w4pin", T=24, H=256, E=6, k=3, I=128, I_s=128, w4=True)
    inp = moe_inputs.generate(wl, seed)
    rng = np.random.default_rng(seed)
    for name in ("w_gate_up_scale", "w_down_scale"):
        exp = rng.integers(-9, -5, size=inp[name].shape)
        sign = rng.choice([-1.0, 1.0], size=inp[name].shape)
        inp[name] = _bf16(sign * np.ldexp(1.0, exp))
    ref = dict(inp)
    for name in ("w_gate_up", "w_down"):
        q, s = ref.pop(name + "_q"), ref.pop(name + "_scale")
        E, R, half = q.shape
        bits = np.empty((E, R, 2 * half), dtype=np.uint16)
        for e in range(E):
            codes = np.empty((R, 2 * half), dtype=np.int64)
            for j in range(4):   # byte j of each 4-byte word: columns j, j + 4
                codes[:, j::8] = q[e][:, j::4] & 15
                codes[:, j + 4::8] = q[e][:, j::4] >> 4
            sv = moe_inputs.bf16_bits_to_f32(s[e])           # [groups, R]
            vals = (codes - 8) * np.repeat(sv.T, 128, axis=1)[:, :2 * half]
            bits[e] = _bf16(vals)
            assert np.array_equal(moe_inputs.bf16_bits_to_f32(bits[e]), vals.astype(np.float32))
        ref[name] = bits
    return wl, inp, ref


def test_w4_layer_equals_bf16_layer_on_exact_weights():
    wl, inp, ref = _w4_exact_pair(3)
    a = mo.forward(inp, k=wl.k, rsf=wl.rsf, limit=wl.limit)
    b = mo.forward(ref, k=wl.k, rsf=wl.rsf, limit=wl.limit)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["y_perm"], b["y_perm"])
    assert np.array_equal(a["out"], b["out"])


def test_w4_scales_make_every_weight_exact_in_bf16():
    """The synthetic scales carry 4 significant bits, so (u - 8) * scale (at
    most 4 + 4 bits) is a bf16 value: the tiled path's bf16 operand equals
    the exact weight."""
    wl = moe_inputs.WORKLOADS["decode_w4"].with_(E=2, H=512, I=256)
    inp = moe_inputs.generate(wl, 1)
    for name in ("w_gate_up", "w_down"):
        s = inp[name + "_scale"]
        assert np.all((s & 0xF) == 0) and np.all(s != 0)
        for e in range(s.shape[0]):
            w = mo.dequant_w4(inp[name + "_q"][e], s[e])
            assert np.array_equal(mo.bf16_to_f64(mo.bf16_round(w)), w)


def test_w4_inputs_spread():
    wl = moe_inputs.WORKLOADS["decode_w4"].with_(E=2, H=512, I=256)
    inp = moe_inputs.generate(wl, 0)
    assert inp["w_gate_up_q"].shape == (2, 512, 256)
    assert inp["w_gate_up_scale"].shape == (2, 4, 512)
    assert inp["w_down_q"].shape == (2, 512, 128)
    assert inp["w_down_scale"].shape == (2, 2, 512)
    w = mo.dequant_w4(inp["w_gate_up_q"][0], inp["w_gate_up_scale"][0])
    assert 0.015 < w.std() < 0.025   # about the bf16 experts' N(0, 0.02)
