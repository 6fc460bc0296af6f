"""Pins of the oracle's W4A16 expert weights.  The pages name the W4A16
expert GEMM and call the routed experts NVFP4 but give no layout; the
format is this library's reading: 4-bit integer codes, an OCP E4M3 scale
byte per row and 128 columns, an fp32 tensor scale per matrix.  Pinned by
hand-worked E4M3 values and dequantisations, torch's own E4M3 decoding of
every byte, a nibble packer written out here, the exactness of every
code-times-scale product in bf16 (brute force), and the special case of
weights exact in bf16, where the W4A16 layer must equal the bf16 layer
(pinned elsewhere) bit for bit."""
import numpy as np
import pytest

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


def test_e4m3_hand_values():
    # byte -> sign | exponent field (4 bits, bias 7) | mantissa (3 bits)
    cases = {
        0x38: 1.0,              # 0 0111 000
        0x39: 1.125,            # 0 0111 001: 1 + 1/8
        0x30: 0.5,              # 0 0110 000
        0x40: 2.0,              # 0 1000 000
        0x77: 240.0,            # 0 1110 111: 1.875 * 2^7
        0x7E: 448.0,            # 0 1111 110: 1.75 * 2^8, the largest value
        0x08: 2.0 ** -6,        # 0 0001 000: the smallest normal
        0x07: 7 * 2.0 ** -9,    # 0 0000 111: the largest subnormal, 7/8 * 2^-6
        0x01: 2.0 ** -9,        # 0 0000 001: the smallest subnormal
        0x00: 0.0,
        0xB8: -1.0,             # 1 0111 000
        0xC0: -2.0,
    }
    got = mo.e4m3_to_f64(np.array(list(cases), dtype=np.uint8))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    neg0 = mo.e4m3_to_f64(np.array([0x80], np.uint8))
    assert neg0[0] == 0.0 and np.signbit(neg0[0])
    assert np.all(np.isnan(mo.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))))


def test_e4m3_every_byte_matches_torch():
    """Library routine: torch's float8_e4m3fn decoding of all 256 bytes."""
    torch = pytest.importorskip("torch")
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = mo.e4m3_to_f64(b)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_code_times_scale_is_always_a_bf16_value():
    """(u - 8) has at most 3 significant bits and an E4M3 value at most 4,
    so every product -- all 16 codes against all 254 non-NaN scale bytes --
    is a bf16 value: a kernel may hand it to the bf16 MFMA unrounded."""
    u = np.arange(16, dtype=np.float64) - 8
    s = mo.e4m3_to_f64(np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8))
    prod = np.outer(u, s)
    assert np.array_equal(mo.bf16_to_f64(mo.bf16_round(prod)), prod)


def test_dequant_hand_example():
    # one row, K = 256: two groups of 128 columns
    q = np.full((1, 128), 0x88, dtype=np.uint8)   # nibble 8 everywhere -> 0
    q[0, 0] = 0x9F     # byte 0 of word 0: columns 0, 4: nibbles 15, 9 -> 7, 1
    q[0, 65] = 0x70    # byte 1 of word 16: columns 129, 133: nibbles 0, 7 -> -8, -1
    q[0, 127] = 0x0F   # byte 3 of word 31: columns 251, 255: nibbles 15, 0 -> 7, -8
    scale = np.array([[0x30], [0xC0]], dtype=np.uint8)   # [groups, rows]: 0.5, -2.0
    w = mo.dequant_w4(q, scale)
    assert w.shape == (1, 256)
    assert w[0, 0] == 3.5 and w[0, 4] == 0.5
    assert w[0, 129] == 16.0 and w[0, 133] == 2.0
    assert w[0, 251] == -14.0 and w[0, 255] == 16.0
    assert np.count_nonzero(w) == 6
    w3 = mo.dequant_w4(q, scale, 0.75)   # the tensor scale multiplies every weight
    assert w3[0, 0] == 2.625 and w3[0, 129] == 12.0 and w3[0, 251] == -10.5


def test_dequant_matches_packer_and_scales():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    R, K = 6, 384
    codes = rng.integers(0, 16, size=(R, K))
    scale = rng.integers(0, 0x7F, size=(K // 128, R)).astype(np.uint8)
    scale |= rng.integers(0, 2, size=scale.shape).astype(np.uint8) << 7
    ts = np.float32(0.0371)
    w = mo.dequant_w4(_pack(codes), scale, ts)
    s = torch.from_numpy(scale.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    for r in range(R):
        for c in range(0, K, 7):
            assert w[r, c] == (codes[r, c] - 8) * s[c // 128, r] * float(ts)


def _w4_exact_pair(seed, scales="full"):
    """A small workload in W4A16 form whose tensor scales are powers of two
    (so every weight (u - 8) * e4m3(s) * 2^j is exact in bf16), and the same
    layer with those weights stored as bf16 (computed here from the codes
    and torch's E4M3 decoding)."""
    torch = pytest.importorskip("torch")
    wl = moe_inputs.Workload("w4pin", T=24, H=256, E=6, k=3, I=128, I_s=128, w4=True,
                             w4_scales=scales)
    inp = moe_inputs.generate(wl, seed)
    rng = np.random.default_rng(seed)
    for name in ("w_gate_up_tscale", "w_down_tscale"):
        inp[name] = np.ldexp(1.0, rng.integers(-12, -8, size=wl.E)).astype(np.float32)
    ref = dict(inp)
    for name in ("w_gate_up", "w_down"):
        q, s = ref.pop(name + "_q"), ref.pop(name + "_scale")
        ts = ref.pop(name + "_tscale")
        E, R, half = q.shape
        bits = np.empty((E, R, 2 * half), dtype=np.uint16)
        for e in range(E):
            codes = np.empty((R, 2 * half), dtype=np.int64)
            for j in range(4):   # byte j of each 4-byte word: columns j, j + 4
                codes[:, j::8] = q[e][:, j::4] & 15
                codes[:, j + 4::8] = q[e][:, j::4] >> 4
            sv = torch.from_numpy(s[e].copy()).view(torch.float8_e4m3fn).float().numpy()
            vals = (codes - 8) * np.repeat(sv.T.astype(np.float64), 128, axis=1)[:, :2 * half]
            vals = vals * float(ts[e])
            bits[e] = _bf16(vals)
            assert np.array_equal(moe_inputs.bf16_bits_to_f32(bits[e]), vals.astype(np.float32))
        ref[name] = bits
    return wl, inp, ref


@pytest.mark.parametrize("scales", ["typical", "full"])
def test_w4_layer_equals_bf16_layer_on_exact_weights(scales):
    wl, inp, ref = _w4_exact_pair(3, scales)
    a = mo.forward(inp, k=wl.k, rsf=wl.rsf, limit=wl.limit)
    b = mo.forward(ref, k=wl.k, rsf=wl.rsf, limit=wl.limit)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["y_perm"], b["y_perm"])
    assert np.array_equal(a["out"], b["out"])


def test_w4_inputs_spread():
    wl = moe_inputs.WORKLOADS["decode_w4"].with_(E=2, H=512, I=256)
    inp = moe_inputs.generate(wl, 0)
    assert inp["w_gate_up_q"].shape == (2, 512, 256)
    assert inp["w_gate_up_scale"].shape == (2, 4, 512) and inp["w_gate_up_scale"].dtype == np.uint8
    assert inp["w_down_q"].shape == (2, 512, 128)
    assert inp["w_down_scale"].shape == (2, 2, 512)
    assert inp["w_gate_up_tscale"].shape == (2,) and inp["w_down_tscale"].dtype == np.float32
    w = mo.dequant_w4(inp["w_gate_up_q"][0], inp["w_gate_up_scale"][0],
                      inp["w_gate_up_tscale"][0])
    assert 0.014 < w.std() < 0.027   # about the bf16 experts' N(0, 0.02)
    # the full-range draw covers every scale byte but the NaNs
    full = moe_inputs.generate(wl.with_(w4_scales="full", H=4096, I=2048), 0)
    seen = np.unique(full["w_gate_up_scale"])
    assert len(seen) == 254 and 0x7F not in seen and 0xFF not in seen
