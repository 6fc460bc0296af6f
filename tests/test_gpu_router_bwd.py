"""Router backward on the GPU (moe_router_backward through the C ABI)
against the oracle's exact gradients, within the fp32 forward-error bounds
of the sums ("bridge.models.beam.modeling_beam", _BeamRouterGatingLinear):
  grad_x (bf16): |gpu - exact| <= (1 + 2^-8) E u sum_e |dL W| + 2^-8 |exact|
  grad_w (fp32): |gpu - exact| <= T u sum_t |dL x|
  grad_b (fp32): |gpu - exact| <= T u sum_t |dL|
with u = 2^-24; contiguous, transposed and expanded (stride-0) gradients,
ragged shapes, the prefill size, an empty batch, and bit-for-bit reruns."""
import numpy as np
import pytest

import moe_inputs
from oracle import moe_oracle as mo
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module")
def tl():
    torch, moe = gh.torch_and_lib()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, moe


def _run(tl, T, H, E, layout, seed=0):
    torch, moe = tl
    rng = np.random.default_rng(seed)
    x = moe_inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    if layout == "expanded":
        dl_host = np.broadcast_to(np.float32(0.37), (T, E))
        dl_dev = torch.full((1, 1), 0.37, dtype=torch.float32, device="cuda").expand(T, E)
    else:
        dl_host = (rng.standard_normal((T, E)) * 0.1).astype(np.float32)
        if layout == "transposed":   # a [E, T] buffer viewed as [T, E]
            dl_dev = gh.dev_f32(torch, np.ascontiguousarray(dl_host.T)).t()
        else:
            dl_dev = gh.dev_f32(torch, dl_host)
    p = moe.make_params(T, H, E, 1, 8, 0, 1.0, 7.0)
    gx = torch.full((max(T, 1), H), 0x7FC0, dtype=torch.int16, device="cuda")
    gw = torch.full((E, H), float("nan"), dtype=torch.float32, device="cuda")
    gb = torch.full((E,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(moe.moe_router_backward_workspace_size(p), 16), dtype=torch.uint8,
                     device="cuda")
    xd, wd = gh.dev_bf16(torch, x), gh.dev_f32(torch, w)
    gh.note(f"router backward T={T} H={H} E={E} {layout} strides={tuple(dl_dev.stride())}")
    moe.moe_router_backward(p, dl_dev, xd, wd, gx, gw, gb, ws)
    torch.cuda.synchronize()
    got = dict(gx=gh.to_bits(gx)[:T], gw=gw.cpu().numpy(), gb=gb.cpu().numpy())
    return got, (dl_host, x, w), (p, dl_dev, xd, wd, gx, gw, gb, ws)


def _check(got, inputs):
    dl, x, w = inputs
    T, E = dl.shape
    ref = mo.router_backward(dl, x, w)
    adl = np.abs(np.asarray(dl, np.float64))
    xf = mo.bf16_to_f64(x)
    # fp32 sum error b, then one bf16 rounding of a value within b of the
    # exact one: at most 2^-8 of its magnitude
    b = E * U * (adl @ np.abs(w.astype(np.float64)))
    bx = (1 + 2.0 ** -8) * b + 2.0 ** -8 * np.abs(ref["grad_x_f64"]) + 1e-37
    dx = np.abs(mo.bf16_to_f64(got["gx"]) - ref["grad_x_f64"])
    assert np.all(dx <= bx), f"grad_x: max d/bound {float((dx / bx).max())}"
    bw = T * U * (adl.T @ np.abs(xf)) + 1e-37
    dw = np.abs(got["gw"].astype(np.float64) - ref["grad_w_f64"])
    assert np.all(dw <= bw), f"grad_w: max d/bound {float((dw / bw).max())}"
    bb = T * U * adl.sum(axis=0) + 1e-37
    db = np.abs(got["gb"].astype(np.float64) - ref["grad_b_f64"])
    assert np.all(db <= bb), f"grad_b: max d/bound {float((db / bb).max())}"
    rep = dict(gx_exact_frac=float(np.mean(got["gx"] == ref["grad_x"])),
               gw_max_d_over_bound=float((dw / bw).max()),
               gx_max_d_over_bound=float((dx / bx).max()))
    gh.note(f"  {rep}")
    return rep


@pytest.mark.parametrize("T,H,E,layout", [
    (300, 520, 24, "contiguous"),     # ragged: H not a multiple of 128, E of 32
    (257, 1032, 300, "transposed"),   # E > 256, strides (1, T)
    (1000, 256, 64, "expanded"),      # the gradient of logits.sum(): strides (0, 0)
    (40, 4096, 64, "contiguous"),     # a decode-sized batch (one token slice)
])
def test_router_backward_parity(tl, T, H, E, layout):
    got, inputs, _ = _run(tl, T, H, E, layout)
    _check(got, inputs)


def test_router_backward_prefill_size_and_rerun(tl):
    torch, moe = tl
    got, inputs, bufs = _run(tl, 8192, 4096, 64, "contiguous", seed=3)
    _check(got, inputs)
    p, dl_dev, xd, wd, gx, gw, gb, ws = bufs
    moe.moe_router_backward(p, dl_dev, xd, wd, gx, gw, gb, ws)
    torch.cuda.synchronize()
    assert np.array_equal(gh.to_bits(gx), got["gx"])
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), got["gw"].view(np.uint32))
    assert np.array_equal(gb.cpu().numpy().view(np.uint32), got["gb"].view(np.uint32))


def test_router_backward_empty_batch(tl):
    torch, moe = tl
    p = moe.make_params(0, 256, 16, 1, 8, 0, 1.0, 7.0)
    gw = torch.full((16, 256), float("nan"), dtype=torch.float32, device="cuda")
    gb = torch.full((16,), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_router_backward(p, None, None, None, None, gw, gb, None)
    torch.cuda.synchronize()
    assert np.all(gw.cpu().numpy() == 0) and np.all(gb.cpu().numpy() == 0)


@pytest.mark.parametrize("want", [("gx",), ("gw",), ("gb",), ("gw", "gb")])
def test_router_backward_output_subsets(tl, want):
    """Each output may be skipped (NULL); the others are unchanged bits."""
    torch, moe = tl
    full, inputs, bufs = _run(tl, 700, 384, 40, "contiguous", seed=9)
    p, dl_dev, xd, wd, gx, gw, gb, ws = bufs
    outs = dict(gx=torch.full_like(gx, 0x7FC0), gw=torch.full_like(gw, float("nan")),
                gb=torch.full_like(gb, float("nan")))
    gh.note(f"router backward subset {want}")
    moe.moe_router_backward(p, dl_dev, xd, wd, *[outs[k] if k in want else None
                                                   for k in ("gx", "gw", "gb")], ws)
    torch.cuda.synchronize()
    if "gx" in want:
        assert np.array_equal(gh.to_bits(outs["gx"])[:700], full["gx"])
    if "gw" in want:
        assert np.array_equal(outs["gw"].cpu().numpy(), full["gw"])
    if "gb" in want:
        # alone, grad_b is summed by its own kernel (another order): check the bound
        _, _, _ = inputs
        dl = inputs[0].astype(np.float64)
        ref = dl.sum(axis=0)
        got = outs["gb"].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref) <= 700 * U * np.abs(dl).sum(axis=0) + 1e-37)
