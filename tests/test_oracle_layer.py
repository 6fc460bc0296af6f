"""Pins for the expert FFN, combine and the layer as a whole (S0, S4-S7):
clamp branches, the E=1 reduction to a library-built SwiGLU FFN, the
dense-mask rendering, the loop rendering, expert-range linearity, row
independence, RMSNorm closed forms and the ScMoE wiring."""
import math

import numpy as np
import pytest
import torch

import moe_inputs
from oracle import loops
from oracle import moe_oracle as mo
from tests.helpers import tiny_inputs


def _widen(u):
    return mo.bf16_to_f64(u)


# ------------------------------------------------------------ clamp ----

def test_clamp_stress_all_four_branches():
    """Large weights push |g|, |u| past L; every branch occurs and each
    element of h follows the branch rule (gate above only, up both sides)."""
    inp = tiny_inputs(T=32, H=16, E=4, k=2, I=24, I_s=8, std=1.5, seed=3)
    L = 7.0
    a = _widen(inp["x"])
    wgu = inp["w_gate_up"][0]
    I = wgu.shape[0] // 2
    g = a @ _widen(wgu[:I]).T
    u = a @ _widen(wgu[I:]).T
    h, _ = mo.swiglu_ffn(a, wgu, inp["w_down"][0], L, round_h=False)
    assert (g > L).sum() > 0 and (g < -L).sum() > 0
    assert (u > L).sum() > 0 and (u < -L).sum() > 0
    for i, j in zip(*np.nonzero(g < -L)):          # not clamped from below
        gg = g[i, j]
        uu = max(-L, min(u[i, j], L))
        assert h[i, j] == pytest.approx(gg / (1 + math.exp(-gg)) * uu, rel=1e-12, abs=1e-300)
    for i, j in zip(*np.nonzero(g > L)):           # clamped from above
        uu = max(-L, min(u[i, j], L))
        assert h[i, j] == pytest.approx(L / (1 + math.exp(-L)) * uu, rel=1e-12)
    m = np.abs(u) > L
    sgn = np.sign(u[m])
    gg = np.minimum(g[m], L)
    np.testing.assert_allclose(h[m], gg / (1 + np.exp(-gg)) * L * sgn, rtol=1e-12)


# ------------------------------------------------ E=1 reduction (torch) ----

def _torch_swiglu_ffn(x64, wgu, wd, L):
    """A textbook clamped SwiGLU FFN in torch float64; h rounded to bf16 by
    torch's own conversion."""
    t = lambda u: torch.from_numpy(moe_inputs.bf16_bits_to_f32(u)).double()
    I = wgu.shape[0] // 2
    W = t(wgu)
    g = x64 @ W[:I].T
    u = x64 @ W[I:].T
    h = torch.nn.functional.silu(torch.clamp(g, max=L)) * torch.clamp(u, -L, L)
    h = h.float().to(torch.bfloat16).double()
    return h @ t(wd).T


@pytest.mark.parametrize("with_shared", [False, True])
def test_single_expert_reduces_to_dense_ffn(with_shared):
    """E=1, k=1, zero router, rsf=2: sigmoid(0)*2 = 1, so the layer is the
    dense clamped SwiGLU FFN (plus the shared FFN when present)."""
    inp = tiny_inputs(T=9, H=24, E=1, k=1, I=16, I_s=12 if with_shared else 0, std=0.6, seed=5)
    inp["w_router"][:] = 0
    inp["corr_bias"][:] = 0
    res = mo.forward(inp, k=1, rsf=2.0, limit=7.0)
    assert np.all(res["w"] == 1.0)
    x64 = torch.from_numpy(moe_inputs.bf16_bits_to_f32(inp["x"])).double()
    ref = _torch_swiglu_ffn(x64, inp["w_gate_up"][0], inp["w_down"][0], 7.0)
    if with_shared:
        ref = ref + _torch_swiglu_ffn(x64, inp["ws_gate_up"], inp["ws_down"], 7.0)
    np.testing.assert_allclose(res["z"], ref.numpy(), rtol=1e-12, atol=1e-12)
    ref_bits = ref.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(res["out"], ref_bits)


def test_single_expert_random_router_scales_by_score():
    """E=1 with a random router: out = rsf*sigmoid(l_t)*FFN0(x_t) + FFN_s(x_t)."""
    inp = tiny_inputs(T=7, H=16, E=1, k=1, I=8, I_s=8, std=0.4, seed=6)
    rsf = 1.75
    res = mo.forward(inp, k=1, rsf=rsf, limit=7.0)
    x64 = torch.from_numpy(moe_inputs.bf16_bits_to_f32(inp["x"])).double()
    f0 = _torch_swiglu_ffn(x64, inp["w_gate_up"][0], inp["w_down"][0], 7.0).numpy()
    fs = _torch_swiglu_ffn(x64, inp["ws_gate_up"], inp["ws_down"], 7.0).numpy()
    l = x64.numpy() @ inp["w_router"][0].astype(np.float64)
    sig = (1 / (1 + np.exp(-l.astype(np.float32).astype(np.float64)))).astype(np.float32)
    w = (np.float32(rsf) * sig).astype(np.float32)
    np.testing.assert_allclose(res["z"], w[:, None].astype(np.float64) * f0 + fs, rtol=1e-12, atol=1e-12)


# ----------------------------------------------- dense-mask rendering ----

@pytest.mark.parametrize("seed", range(3))
def test_dense_mask_rendering_equals_permuted(seed):
    """Run every expert on every token and weight by a T x E selection mask;
    no permutation involved.  Must equal the permute-based combine."""
    inp = tiny_inputs(T=20, H=16, E=6, k=3, I=8, I_s=5, std=0.4, seed=seed)
    res = mo.forward(inp, k=3, rsf=1.3, limit=7.0)
    T, E = 20, 6
    mask = np.zeros((T, E))
    for t in range(T):
        for j, e in enumerate(res["ids"][t]):
            mask[t, e] = float(res["w"][t, j])
    a = _widen(inp["x"])
    z = mo.swiglu_ffn(a, inp["ws_gate_up"], inp["ws_down"], 7.0)[1]
    for e in range(E):
        z = z + mask[:, e:e + 1] * mo.swiglu_ffn(a, inp["w_gate_up"][e], inp["w_down"][e], 7.0)[1]
    np.testing.assert_allclose(res["z"], z, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------ loop rendering ----

@pytest.mark.parametrize("seed", range(4))
def test_loop_rendering_agrees(seed):
    inp = tiny_inputs(T=6, H=8, E=5, k=2, I=4, I_s=3, std=0.9, seed=seed)
    res = mo.forward(inp, k=2, rsf=2.5, limit=7.0)
    W = lambda u: moe_inputs.bf16_bits_to_f32(u).astype(np.float64).tolist()
    lp = loops.forward_loops(
        W(inp["x"]), inp["w_router"].astype(np.float64).tolist(),
        inp["corr_bias"].astype(np.float64).tolist(),
        W(inp["w_gate_up"]), W(inp["w_down"]), W(inp["ws_gate_up"]), W(inp["ws_down"]),
        k=2, rsf=2.5, L=7.0)
    assert res["ids"].tolist() == lp["ids"]
    assert res["w"].astype(np.float64).tolist() == lp["w"]
    assert res["offsets"].tolist() == lp["offsets"]
    assert res["sorted_token"].tolist() == lp["sorted_token"]
    assert res["inv_pos"].tolist() == lp["inv_pos"]
    np.testing.assert_allclose(res["z"], np.array(lp["z"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(_widen(res["out"]), np.array(lp["out"]))


# ------------------------------------------- expert-range linearity ----

def test_expert_ranges_partition_sums_to_full():
    """Split the experts into disjoint ranges (one per expert-parallel rank);
    each partial holds its experts' slots, the shared expert goes into
    exactly one partial.  The partials sum to the full combine."""
    inp = tiny_inputs(T=30, H=16, E=8, k=3, I=8, I_s=6, std=0.4, seed=11)
    kw = dict(k=3, rsf=1.2, limit=7.0)
    full = mo.forward(inp, **kw)
    ranges = [(0, 2), (2, 5), (5, 6), (6, 8)]
    parts = [mo.forward(inp, expert_range=r, include_shared=(i == 0), **kw)["z"]
             for i, r in enumerate(ranges)]
    np.testing.assert_allclose(sum(parts), full["z"], rtol=1e-12, atol=1e-12)
    # adding the shared expert on every rank is caught
    twice = sum(mo.forward(inp, expert_range=r, **kw)["z"] for r in ranges)
    assert np.abs(twice - full["z"]).max() > 1e-3


def test_rsf_scales_routed_part_only():
    inp = tiny_inputs(T=12, H=16, E=6, k=2, I=8, I_s=6, std=0.4, seed=12)
    a = mo.forward(inp, k=2, rsf=1.0, limit=7.0)
    b = mo.forward(inp, k=2, rsf=2.0, limit=7.0)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_allclose(b["z"] - b["ys"], 2 * (a["z"] - a["ys"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(a["ys"], b["ys"])


def test_row_independence():
    inp = tiny_inputs(T=24, H=16, E=6, k=2, I=8, I_s=6, std=0.4, seed=13)
    kw = dict(k=2, rsf=1.0, limit=7.0)
    full = mo.forward(inp, **kw)
    perm = np.random.default_rng(0).permutation(24)
    sh = mo.forward(mo.take_rows(inp, perm), **kw)
    np.testing.assert_array_equal(sh["ids"], full["ids"][perm])
    np.testing.assert_array_equal(sh["out"], full["out"][perm])
    half = mo.forward(mo.take_rows(inp, np.arange(12, 24)), **kw)
    np.testing.assert_array_equal(half["out"], full["out"][12:])


# ------------------------------------------------------------ RMSNorm ----

def test_rmsnorm_closed_form():
    v = mo.rmsnorm_f64(np.array([[3.0, 4.0]]), None, 0.0)
    np.testing.assert_allclose(v, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)
    np.testing.assert_allclose(v, [[0.8485281, 1.1313708]], rtol=1e-7)
    xb = moe_inputs.f32_to_bf16_bits(np.array([[3.0, 4.0]], np.float32))
    got = mo.bf16_to_f64(mo.rmsnorm_bf16(xb, None, 0.0))
    # bf16 neighbours of 0.8485 are 0.84765625 and 0.8515625; of 1.1314: 1.125 and 1.1328125
    np.testing.assert_array_equal(got, [[0.84765625, 1.1328125]])


def test_rmsnorm_gain_closed_form():
    """RMSNorm([3, 4]) with gain [2, 1/2], worked by hand: r = 1/sqrt(12.5),
    so the values are 6r = 1.6970563 and 2r = 0.5656854.  bf16 keeps 8
    significant bits: in [1, 2) the step is 2^-7, and 1.6970563 lies between
    1.6953125 (217 steps) and 1.703125 (218), nearer the first; in [1/2, 1)
    the step is 2^-8, and 0.5656854 lies between 0.5625 (144 steps) and
    0.56640625 (145), nearer the second.  Ignoring the gain would give
    [0.84765625, 1.1328125], dividing by it [0.423828125, 2.265625]."""
    xb = moe_inputs.f32_to_bf16_bits(np.array([[3.0, 4.0]], np.float32))
    g = np.array([2.0, 0.5], np.float32)
    got = mo.bf16_to_f64(mo.rmsnorm_bf16(xb, g, 0.0))
    np.testing.assert_array_equal(got, [[1.6953125, 0.56640625]])


def test_scmoe_pre_gain_scales_routed_input_per_channel():
    """The ScMoE pre-norm gain multiplies each channel of the routed input:
    a power-of-two gain on one channel scales exactly that column of xr by
    the same power of two (bf16 rounding commutes with it) and leaves the
    others and the shared path alone; the post-norm gain does not touch xr."""
    H = 32
    inp = tiny_inputs(T=16, H=H, E=6, k=2, I=8, I_s=8, std=0.3, seed=23, scmoe=True)
    kw = dict(k=2, rsf=1.0, limit=7.0, scmoe=True, eps=1e-6)
    base = mo.forward(inp, **kw)
    for ch, c in ((0, 4.0), (7, 0.25), (31, 2.0)):
        g = np.ones(H, np.float32)
        g[ch] = c
        got = mo.forward(dict(inp, gamma_pre=g), **kw)
        xb, xg = mo.bf16_to_f64(base["xr"]), mo.bf16_to_f64(got["xr"])
        np.testing.assert_array_equal(xg[:, ch], c * xb[:, ch])
        others = np.arange(H) != ch
        np.testing.assert_array_equal(xg[:, others], xb[:, others])
        np.testing.assert_array_equal(got["ys"], base["ys"])
    # the post-norm gain leaves the routed input alone
    gp = np.linspace(0.5, 1.5, H).astype(np.float32)
    np.testing.assert_array_equal(mo.forward(dict(inp, gamma_post=gp), **kw)["xr"], base["xr"])


def test_scmoe_routes_the_gained_input():
    """With a jittered pre-norm gain the routed half of the ScMoE layer is
    the plain layer run on the gained, normalised input: a gain of 2^j on
    every channel gives xr exactly 2^j times the unit-gain xr, and the
    router then sees logits 2^j times larger."""
    H = 32
    inp = tiny_inputs(T=16, H=H, E=6, k=2, I=8, I_s=8, std=0.3, seed=24, scmoe=True)
    kw = dict(k=2, rsf=1.0, limit=7.0, scmoe=True, eps=1e-6)
    base = mo.forward(inp, **kw)
    four = mo.forward(dict(inp, gamma_pre=np.full(H, 4.0, np.float32)), **kw)
    np.testing.assert_array_equal(mo.bf16_to_f64(four["xr"]), 4.0 * mo.bf16_to_f64(base["xr"]))
    np.testing.assert_allclose(four["logits"], 4.0 * base["logits"], rtol=1e-6, atol=1e-7)
    g = (1 + np.random.default_rng(3).uniform(-0.1, 0.1, H)).astype(np.float32)
    a = mo.forward(dict(inp, gamma_pre=g), **kw)
    c = mo.forward(dict(inp, x=a["xr"]), k=2, rsf=1.0, limit=7.0, include_shared=False)
    np.testing.assert_array_equal(a["ids"], c["ids"])
    np.testing.assert_allclose(a["z"] - a["ys"], c["z"], rtol=1e-12, atol=1e-12)


def test_rmsnorm_scale_invariance_exact_for_powers_of_two():
    rng = np.random.default_rng(4)
    x = moe_inputs.f32_to_bf16_bits(rng.standard_normal((5, 64)).astype(np.float32))
    x2 = moe_inputs.f32_to_bf16_bits(2 * moe_inputs.bf16_bits_to_f32(x))
    g = rng.uniform(0.9, 1.1, 64).astype(np.float32)
    np.testing.assert_array_equal(mo.rmsnorm_bf16(x, g, 0.0), mo.rmsnorm_bf16(x2, g, 0.0))


def test_rmsnorm_unit_rms_and_eps():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((6, 40)) * 7
    v = mo.rmsnorm_f64(z, None, 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(v * v, axis=1)), 1.0, rtol=1e-6)
    # eps matters for a row of zeros: 0 / sqrt(eps) = 0, no NaN
    assert np.all(mo.rmsnorm_f64(np.zeros((1, 4)), None, 1e-6) == 0)


# -------------------------------------------------------------- ScMoE ----

def test_scmoe_wiring():
    """Routed path sees only RMSNorm(x_prev); the shared expert only x_cur;
    the post-norm acts on the merged sum."""
    inp = tiny_inputs(T=16, H=32, E=6, k=2, I=8, I_s=8, std=0.3, seed=21, scmoe=True)
    kw = dict(k=2, rsf=1.0, limit=7.0, scmoe=True, eps=1e-6)
    a = mo.forward(inp, **kw)
    # 1) a different x_cur changes only the shared term
    inp2 = dict(inp, x_cur=moe_inputs.generate(moe_inputs.Workload(
        "t", T=16, H=32, E=6, k=2, I=8, I_s=8, scmoe=True), seed=99)["x_cur"])
    b = mo.forward(inp2, **kw)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_array_equal(a["y_perm"], b["y_perm"])
    np.testing.assert_array_equal(a["w"], b["w"])
    np.testing.assert_allclose(a["z"] - a["ys"], b["z"] - b["ys"], rtol=1e-12, atol=1e-12)
    assert np.abs(a["ys"] - b["ys"]).max() > 0
    # 2) the routed part equals the plain layer run on xr
    plain_inp = dict(inp, x=a["xr"])
    c = mo.forward(plain_inp, k=2, rsf=1.0, limit=7.0, include_shared=False)
    np.testing.assert_array_equal(a["ids"], c["ids"])
    np.testing.assert_allclose(a["z"] - a["ys"], c["z"], rtol=1e-12, atol=1e-12)
    # 3) the output rows have unit RMS before rounding (gamma_post = 1)
    np.testing.assert_allclose(np.sqrt(np.mean(a["out_f64"] ** 2, axis=1)), 1.0, rtol=1e-5)


def test_scmoe_gamma_applied_per_channel():
    inp = tiny_inputs(T=4, H=16, E=4, k=1, I=8, I_s=8, std=0.3, seed=22, scmoe=True)
    kw = dict(k=1, rsf=1.0, limit=7.0, scmoe=True, eps=1e-6)
    a = mo.forward(inp, **kw)
    g = np.linspace(0.5, 1.5, 16).astype(np.float32)
    b = mo.forward(dict(inp, gamma_post=g), **kw)
    np.testing.assert_allclose(b["out_f64"], a["out_f64"] * g.astype(np.float64), rtol=1e-12)
