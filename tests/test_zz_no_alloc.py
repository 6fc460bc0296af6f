"""moe_forward_noalloc (the layer on the library's fixed device scratch)
against moe_forward on the same inputs, through the C ABI: two calls in a
row on one device, the second with a smaller batch, each compared bit for
bit with moe_forward and with the oracle at the layer's parity bar; the
same with the tile-blocked expert copies and h left unprobed (the blocked
layouts of the 256-row tiles); and a batch too large for the scratch
rejected before anything is enqueued."""
import numpy as np
import pytest

import moe_inputs
from moe_inputs import Workload
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

# a layer with a shared expert; 2400 tokens (600 routed rows per expert)
# take the 256-row pipelined tiles, 600 tokens the 128-row ones, 40 tokens
# the weight-streaming ones (where moe_forward runs the shared expert on
# its second stream and the fixed-scratch call does not)
LAYER = Workload("noalloc", T=2400, H=256, E=8, k=2, I=160, I_s=96, rsf=1.3)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch, _ = gh.torch_and_lib()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _compare(T, packed=False):
    torch, moe = gh.torch_and_lib()
    inp = moe_inputs.generate(LAYER, seed=11, T=T)
    gh.note(f"noalloc vs moe_forward {LAYER.label()} T={T} packed={packed}")
    d = gh.Device(LAYER, inp)
    d.canary()
    d.run()
    ref = d.result()
    if packed:  # the checked reference above keeps the row-major weights and probes h
        d.pack()
        d.unprobe_h()
    d.canary()
    moe.moe_forward_noalloc(d.params, d.x, d.x_cur, d.weights, d.out, d.probes)
    got = d.result()
    for key in ("out", "ids", "w", "offsets", "sorted_token", "inv_pos", "logits"):
        assert np.array_equal(got[key], ref[key], equal_nan=True), f"{key} differs (T={T})"
    rep = gh.check_layer(LAYER, inp, ref)
    gh.note(f"  {rep}")
    assert rep["rows_checked"] == T


def test_noalloc_matches_forward_twice_second_smaller():
    _compare(2400)
    _compare(600)
    _compare(40)


def test_noalloc_with_blocked_layouts():
    _compare(2400, packed=True)
    _compare(600, packed=True)


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    torch, moe = gh.torch_and_lib()
    T, H, E, k, I = 8192, 4096, 64, 8, 1536
    p = moe.make_params(T, H, E, k, I, 0, 1.0, 7.0)
    assert moe.moe_workspace_size(p) > moe.MOE_NOALLOC_SCRATCH_BYTES
    # tiny stand-ins: the size check comes before any pointer is used
    x = torch.zeros(16, dtype=torch.int16, device="cuda")
    out = torch.full((16,), 0x7FC0, dtype=torch.int16, device="cuda")
    w = moe.make_weights(torch.zeros(16, device="cuda"), None, x, x)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(p, x, None, w, out)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    assert "fixed scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0x7FC0)
