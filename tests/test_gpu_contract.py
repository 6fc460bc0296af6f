"""The C ABI's contract on the GPU (the conventions stated at the top of
include/moe.h): identical inputs give identical bits; a call that returns
an error enqueues nothing and touches no output; no kernel writes outside
the buffers it was given (guard bytes around the workspace and the output
stay intact); work runs on the caller's stream; two host threads may call
the library at once, each on its own stream."""
import threading

import numpy as np
import pytest

import moe_inputs
from moe_inputs import Workload
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

CASES = {
    "decode_small": Workload("c_decode", T=20, H=512, E=40, k=4, I=176, I_s=352),
    "prefill_small": Workload("c_prefill", T=600, H=256, E=4, k=2, I=160, I_s=96),
    "scmoe": Workload("c_scmoe", T=120, H=384, E=32, k=4, I=192, I_s=256, scmoe=True,
                      gamma_jitter=0.1),
    "w4_decode": Workload("c_w4", T=40, H=512, E=16, k=4, I=384, I_s=256, w4=True),
    "w4_prefill": Workload("c_w4p", T=600, H=256, E=4, k=2, I=256, I_s=128, w4=True),
}


@pytest.fixture(scope="module")
def tl():
    torch, moe = gh.torch_and_lib()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, moe


@pytest.mark.parametrize("name", list(CASES))
def test_repeated_calls_are_bit_identical(tl, name):
    wl = CASES[name]
    inp = moe_inputs.generate(wl, seed=2)
    gh.note(f"determinism {name}")
    d = gh.Device(wl, inp)
    outs = []
    for _ in range(3):
        d.canary()
        d.run()
        outs.append(d.result())
    for r in outs[1:]:
        for key in ("out", "ids", "w", "offsets", "sorted_token", "inv_pos", "logits"):
            assert np.array_equal(np.asarray(r[key]).view(np.uint8),
                                  np.asarray(outs[0][key]).view(np.uint8)), key


def test_error_leaves_outputs_untouched(tl):
    torch, moe = tl
    wl = CASES["decode_small"]
    inp = moe_inputs.generate(wl, seed=3)
    d = gh.Device(wl, inp)
    d.canary()
    torch.cuda.synchronize()
    before = gh.to_bits(d.out).copy()
    bad = [
        moe.make_params(wl.T, wl.H, wl.E, 0, wl.I, wl.I_s, wl.rsf, wl.limit),        # k = 0
        moe.make_params(wl.T, wl.H, wl.E, wl.k, wl.I, wl.I_s, wl.rsf, float("nan")),  # no limit
    ]
    for p in bad:
        with pytest.raises(moe.MoeError):
            moe.moe_forward(p, d.x, None, d.weights, d.out, d.probes, d.ws)
    short = d.ws[: d.ws.numel() // 2]
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward(d.params, d.x, None, d.weights, d.out, d.probes, short)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert np.array_equal(gh.to_bits(d.out), before)
    assert np.all(d.ids.cpu().numpy() == -7)   # the canary of the probe outputs


@pytest.mark.parametrize("name", ["decode_small", "prefill_small", "scmoe", "w4_prefill"])
def test_no_write_outside_the_buffers(tl, name):
    """Workspace and output carved out of larger buffers whose guard bytes
    before and after must survive the call."""
    torch, moe = tl
    wl = CASES[name]
    inp = moe_inputs.generate(wl, seed=4)
    d = gh.Device(wl, inp)
    G = 4096  # guard bytes (a multiple of 256 keeps the alignment)
    need = moe.moe_workspace_size(d.params)
    ws_all = torch.full((need + 2 * G,), 0xA5, dtype=torch.uint8, device="cuda")
    out_all = torch.full((wl.T * wl.H + 2 * G // 2,), 0x5A5A, dtype=torch.int16, device="cuda")
    ws = ws_all[G:G + need]
    out = out_all[G // 2:G // 2 + wl.T * wl.H].view(wl.T, wl.H)
    gh.note(f"guards {name} ws={need}")
    moe.moe_forward(d.params, d.x, d.x_cur, d.weights, out, d.probes, ws)
    torch.cuda.synchronize()
    w = ws_all.cpu().numpy()
    o = out_all.cpu().numpy()
    assert np.all(w[:G] == 0xA5) and np.all(w[G + need:] == 0xA5)
    assert np.all(o[:G // 2] == 0x5A5A) and np.all(o[G // 2 + wl.T * wl.H:] == 0x5A5A)
    d.canary()
    d.run()
    assert np.array_equal(gh.to_bits(out), d.result()["out"])


def test_runs_on_the_callers_stream(tl):
    torch, moe = tl
    wl = CASES["decode_small"]
    inp = moe_inputs.generate(wl, seed=5)
    d = gh.Device(wl, inp)
    d.run()
    ref = d.result()["out"]
    s = torch.cuda.Stream()
    out = torch.full_like(d.out, 0x7FC0)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        moe.moe_forward(d.params, d.x, None, d.weights, out, None, d.ws)
    s.synchronize()   # the call's work is ordered on s alone
    assert np.array_equal(gh.to_bits(out), ref)


def test_two_threads_at_once(tl):
    """Two host threads, each with its own stream, inputs and workspace,
    call moe_forward repeatedly at the same time; both results stay exact."""
    torch, moe = tl
    devs, refs = [], []
    for name in ("decode_small", "w4_decode"):
        wl = CASES[name]
        d = gh.Device(wl, moe_inputs.generate(wl, seed=6))
        d.run()
        refs.append(d.result()["out"])
        devs.append(d)
    errors = []

    def worker(i):
        try:
            d = devs[i]
            s = torch.cuda.Stream()
            out = torch.empty_like(d.out)
            with torch.cuda.stream(s):
                for _ in range(20):
                    moe.moe_forward(d.params, d.x, d.x_cur, d.weights, out, None, d.ws)
            s.synchronize()
            if not np.array_equal(gh.to_bits(out), refs[i]):
                errors.append(f"thread {i}: output differs")
        except Exception as e:  # reported below
            errors.append(f"thread {i}: {e!r}")

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
