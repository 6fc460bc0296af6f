"""Pins of the oracle's router backward (gradients of l = x W_r^T + b,
"bridge.models.beam.modeling_beam", _BeamRouterGatingLinear): PyTorch
autograd on the same function in float64, the adjoint identity that ties
the three gradients to the forward, and closed forms for one-hot and
expanded (stride-0) upstream gradients."""
import numpy as np
import torch

import moe_inputs
from oracle import moe_oracle as mo


def _case(T=13, H=40, E=7, seed=0):
    rng = np.random.default_rng(seed)
    x = moe_inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    dl = rng.standard_normal((T, E)).astype(np.float32)
    return x, w, dl


def test_matches_torch_autograd():
    x, w, dl = _case()
    xt = torch.tensor(mo.bf16_to_f64(x), dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    bt = torch.zeros(w.shape[0], dtype=torch.float64, requires_grad=True)
    (xt @ wt.T + bt).backward(torch.tensor(dl, dtype=torch.float64))
    r = mo.router_backward(dl, x, w)
    assert np.allclose(r["grad_x_f64"], xt.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(r["grad_w_f64"], wt.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(r["grad_b_f64"], bt.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.array_equal(r["grad_x"], mo.bf16_round(xt.grad.numpy()))


def test_adjoint_identity():
    # <dL, x W^T> = <grad_w, W> = <grad_x, x> (exact arithmetic)
    x, w, dl = _case(T=31, H=64, E=9, seed=1)
    r = mo.router_backward(dl, x, w)
    xf = mo.bf16_to_f64(x)
    lhs = np.sum(dl.astype(np.float64) * (xf @ w.astype(np.float64).T))
    assert np.isclose(lhs, np.sum(r["grad_w_f64"] * w), rtol=1e-12)
    assert np.isclose(lhs, np.sum(r["grad_x_f64"] * xf), rtol=1e-12)


def test_one_hot_gradient():
    # dL = one-hot rows (token t -> expert e_t): grad_x[t] = W[e_t] exactly
    # (then bf16), grad_w[e] = sum of the x rows of its tokens, grad_b =
    # token counts
    x, w, _ = _case(T=10, H=24, E=4, seed=2)
    e_of = np.array([0, 3, 3, 1, 0, 2, 3, 1, 1, 0])
    dl = np.zeros((10, 4), np.float32)
    dl[np.arange(10), e_of] = 1.0
    r = mo.router_backward(dl, x, w)
    assert np.array_equal(r["grad_x_f64"], w[e_of].astype(np.float64))
    xf = mo.bf16_to_f64(x)
    for e in range(4):
        assert np.array_equal(r["grad_w_f64"][e], xf[e_of == e].sum(axis=0))
    assert r["grad_b"].tolist() == [3.0, 3.0, 1.0, 3.0]


def test_expanded_gradient():
    # the gradient of logits.sum() is an expanded (stride-0) array of ones
    x, w, _ = _case(T=17, H=32, E=5, seed=3)
    dl = np.broadcast_to(np.float32(0.5), (17, 5))
    assert dl.strides == (0, 0)
    r = mo.router_backward(dl, x, w)
    xf = mo.bf16_to_f64(x)
    assert np.allclose(r["grad_x_f64"], 0.5 * np.tile(w.astype(np.float64).sum(0), (17, 1)), rtol=1e-14)
    assert np.allclose(r["grad_w_f64"], 0.5 * np.tile(xf.sum(0), (5, 1)), rtol=1e-14)
    assert r["grad_b"].tolist() == [8.5] * 5
