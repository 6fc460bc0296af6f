"""Whole-layer parity on the GPU (moe_forward through the C ABI) against
the oracle: small and medium shapes compared on every element, the
measured workloads at full size on every token's routing, permutation and
output (a few variant runs check a sample of tokens' outputs: the layer is
row-independent, so the oracle computes those rows alone), plus the layer's
degenerate cases."""
import numpy as np
import pytest

import moe_inputs
from moe_inputs import Workload
from oracle import moe_oracle as mo
from tests import gpu_harness as gh
from tests.helpers import load_hand_example

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch, _ = gh.torch_and_lib()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_and_check(wl, inp, rows=None):
    gh.note(f"forward {wl.label()} T={inp['x'].shape[0]}")
    d = gh.Device(wl, inp)
    d.canary()
    d.run()
    gpu = d.result()
    rep = gh.check_layer(wl, inp, gpu, rows)
    gh.note(f"  {rep}")
    return rep, gpu, d


SMALL = {
    "tiny": moe_inputs.WORKLOADS["tiny"],
    # several m-tiles and n-tiles, K and N tails (H, I not multiples of 64/128)
    "medium_ragged": Workload("medium_ragged", T=300, H=520, E=24, k=6, I=264, I_s=136, rsf=1.7),
    # decode-like: few rows per expert (weight-streaming tiles)
    "decode_small": Workload("decode_small", T=20, H=512, E=40, k=4, I=176, I_s=352),
    # no shared expert
    "no_shared": Workload("no_shared", T=150, H=256, E=16, k=3, I=128, I_s=0),
    # clamp stress: large weights push |g|, |u| past the limit
    "clamp_stress": Workload("clamp_stress", T=64, H=128, E=8, k=2, I=256, I_s=256,
                             weight_std=0.3),
    # ScMoE pairing with random RMSNorm gains
    "scmoe_gamma": Workload("scmoe_gamma", T=200, H=384, E=32, k=4, I=192, I_s=256,
                            scmoe=True, gamma_jitter=0.1),
    # k at its bound, many experts
    "k16": Workload("k16", T=96, H=256, E=300, k=16, I=64, I_s=64, rsf=2.5),
    # long expert segments (LDS-tiled GEMM variant), several m-tiles per expert
    "prefill_small": Workload("prefill_small", T=520, H=256, E=8, k=2, I=200, I_s=136),
    # long segments with H, I multiples of 32 (the pipelined tiles apply):
    # ragged last m-tile, an N tail in gate_up (I = 160 < 2 x 128)
    "pipe_small": Workload("pipe_small", T=600, H=256, E=4, k=2, I=160, I_s=96, rsf=1.3),
    # decode-like, weight-streaming tiles: whole 256-wide K stages in gate_up,
    # a partial last stage in down (I = 384)
    "stream_small": Workload("stream_small", T=40, H=512, E=16, k=4, I=384, I_s=256),
    # weight streaming with segments of several 32-row m-tiles and both
    # 16-row halves; partial K stages in gate_up (H = 384) and in the shared
    # down projection (a single half stage, I_s = 128)
    "stream_multi": Workload("stream_multi", T=300, H=384, E=8, k=2, I=256, I_s=128, rsf=1.5),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    wl = SMALL[name]
    inp = moe_inputs.generate(wl, seed=0)
    rep, _, _ = run_and_check(wl, inp)
    assert rep["rows_checked"] == wl.T


def test_forward_hand_example():
    inp, p, exp = load_hand_example()
    # the library needs H, I multiples of 8: embed the example in zeros
    H8, I8 = 8, 8
    T, E = p["T"], p["E"]
    x = np.zeros((T, H8), np.uint16)
    x[:, :2] = inp["x"]
    wr = np.zeros((E, H8), np.float32)
    wr[:, :2] = inp["w_router"]
    wgu = np.zeros((E, 2 * I8, H8), np.uint16)
    wgu[:, 0, :2] = inp["w_gate_up"][:, 0]
    wgu[:, I8, :2] = inp["w_gate_up"][:, 1]
    wd = np.zeros((E, H8, I8), np.uint16)
    wd[:, :2, 0] = inp["w_down"][:, :, 0]
    sgu = np.zeros((2 * I8, H8), np.uint16)
    sgu[0, :2] = inp["ws_gate_up"][0]
    sgu[I8, :2] = inp["ws_gate_up"][1]
    sd = np.zeros((H8, I8), np.uint16)
    sd[:2, 0] = inp["ws_down"][:, 0]
    full = dict(x=x, w_router=wr, corr_bias=inp["corr_bias"], w_gate_up=wgu, w_down=wd,
                ws_gate_up=sgu, ws_down=sd)
    wl = Workload("hand", T=T, H=H8, E=E, k=p["k"], I=I8, I_s=I8, rsf=p["rsf"], limit=p["limit"])
    rep, gpu, _ = run_and_check(wl, full)
    np.testing.assert_array_equal(gpu["ids"], exp["ids"])
    np.testing.assert_array_equal(gpu["offsets"], exp["offsets"])
    np.testing.assert_array_equal(gpu["sorted_token"], exp["sorted_token"])
    np.testing.assert_array_equal(gpu["inv_pos"], exp["inv_pos"])
    np.testing.assert_allclose(gpu["w"], exp["w"], rtol=1e-7)
    out = mo.bf16_to_f64(gpu["out"][:, :2])
    np.testing.assert_array_equal(out, np.asarray(exp["out"], np.float64))
    assert np.all(gpu["out"][:, 2:] == 0)


def test_forward_single_expert_is_dense_ffn():
    """E=1, k=1, zero router, rsf=2 -> weight exactly 1: the layer is the
    dense clamped SwiGLU FFN plus the shared one."""
    wl = Workload("e1", T=77, H=256, E=1, k=1, I=136, I_s=64, rsf=2.0, weight_std=0.2)
    inp = moe_inputs.generate(wl, seed=3)
    inp["w_router"][:] = 0
    inp["corr_bias"][:] = 0
    rep, gpu, _ = run_and_check(wl, inp)
    assert np.all(gpu["w"] == 1.0)
    assert np.all(gpu["ids"] == 0)


def test_forward_single_token_and_empty_batch():
    wl = Workload("t1", T=1, H=64, E=4, k=2, I=32, I_s=16)
    run_and_check(wl, moe_inputs.generate(wl, seed=1))
    # T = 0 is a no-op that succeeds
    torch, moe = gh.torch_and_lib()
    p = moe.make_params(0, 64, 4, 2, 32, 16, 1.0, 7.0)
    w = moe.make_weights(None, None, None, None)
    out = torch.empty(0, dtype=torch.int16, device="cuda")
    moe.moe_forward(p, None, None, w, out, None, None)


# ---------------------------------------------- measured workloads ----

def _full(name, sample):
    wl = moe_inputs.WORKLOADS[name]
    gh.note(f"generating {wl.label()}")
    inp = moe_inputs.generate(wl, seed=0)
    rows = None
    if sample is not None:
        rows = np.sort(np.random.default_rng(7).choice(wl.T, size=sample, replace=False))
    rep, _, dev = run_and_check(wl, inp, rows)
    del dev
    return rep


def test_forward_decode_full():
    rep = _full("decode", None)
    assert rep["rows_checked"] == 32


def test_forward_prefill_full():
    rep = _full("prefill", None)
    assert rep["rows_checked"] == 8192


def test_forward_scmoe_full():
    rep = _full("scmoe", None)
    assert rep["rows_checked"] == 8192


def test_forward_zipf_full():
    rep = _full("zipf", None)
    assert rep["rows_checked"] == 16384
    # the Zipf-scaled router leaves the expert load strongly skewed
    assert rep["max_over_mean_count"] > 4


@pytest.mark.parametrize("variant", ["wstream", "tile32", "tile128", "pipe256w8", "pingpong"])
@pytest.mark.parametrize("name", ["medium_ragged", "decode_small", "scmoe_gamma", "prefill_small",
                                  "pipe_small", "stream_small", "stream_multi"])
def test_forward_every_tile_variant(monkeypatch, variant, name):
    """Each grouped-GEMM tile variant (forced through MOE_GEMM_VARIANT) gives
    a parity-green layer; the automatic choice is only a speed decision."""
    monkeypatch.setenv("MOE_GEMM_VARIANT", variant)
    wl = SMALL[name]
    step = {"pipe256w8": 32, "pingpong": 32, "wstream": 32}.get(variant)
    if step and (wl.H % step or wl.I % step or wl.I_s % step):
        pytest.skip(f"the pipelined tiles step K in whole {step}-wide stages")
    run_and_check(wl, moe_inputs.generate(wl, seed=1))


@pytest.mark.parametrize("name", ["decode_small", "stream_small"])
def test_forward_graph_replay_matches_eager(name):
    """moe_forward captured into a HIP graph (the weight-streaming path forks
    the shared expert onto a second stream and joins it back) replays to the
    eager result, bit for bit, several times with eager work in between."""
    torch, moe = gh.torch_and_lib()
    wl = SMALL[name]
    gh.note(f"graph replay {wl.label()}")
    d = gh.Device(wl, moe_inputs.generate(wl, seed=2))
    d.run()  # eager, outside the capture (also creates the second stream)
    eager = gh.to_bits(d.out).copy()
    out_g = torch.empty_like(d.out)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_forward(d.params, d.x, d.x_cur, d.weights, out_g, None, d.ws)  # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        moe.moe_forward(d.params, d.x, d.x_cur, d.weights, out_g, None, d.ws)
    for rep in range(3):
        out_g.fill_(0x7FC0)
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gh.to_bits(out_g), eager, err_msg=f"replay {rep}")
        d.run()  # eager work between replays
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gh.to_bits(d.out), eager)


# ------------------------------------------ tile-blocked expert copies ----

def packed_layout(w: np.ndarray, N: int, K: int, gateup: bool) -> np.ndarray:
    """The tile-blocked layout of moe_pack_experts as the header defines it,
    built by indexing: blocks (e, b, s) of 256 rows x 32 values; gate_up tile
    b holds gate rows 128 b + r then up rows N + 128 b + r, down tile b rows
    256 b + r; rows past N zero."""
    E = w.shape[0]
    tile = 128 if gateup else 256
    nt = -(-N // tile)
    out = np.zeros((E, nt, K // 32, 256, 32), dtype=w.dtype)
    for b in range(nt):
        for r in range(256):
            n = tile * b + (r % 128 if gateup else r)
            if n < N:
                src = N + n if gateup and r >= 128 else n
                out[:, b, :, r, :] = w[:, src, :].reshape(E, K // 32, 32)
    return out.reshape(-1)


def test_pack_experts_layout():
    """moe_pack_experts writes every element of the layout, bit for bit:
    ragged tiles in both projections (I = 160 < 2 x 128, H = 288 < 2 x 256)."""
    torch, moe = gh.torch_and_lib()
    E, H, I = 3, 288, 160
    rng = np.random.default_rng(11)
    wgu = rng.integers(0, 1 << 16, size=(E, 2 * I, H), dtype=np.uint16)
    wdn = rng.integers(0, 1 << 16, size=(E, H, I), dtype=np.uint16)
    p = moe.make_params(64, H, E, 2, I, 0, 1.0, 7.0, False, 1e-6)
    gu_n, dn_n = moe.moe_packed_experts_size(p)
    gu = torch.full((gu_n,), 0x7FC0, dtype=torch.int16, device="cuda")
    dn = torch.full((dn_n,), 0x7FC0, dtype=torch.int16, device="cuda")
    gh.note(f"pack E={E} H={H} I={I}")
    moe.moe_pack_experts(p, gh.dev_bf16(torch, wgu), gh.dev_bf16(torch, wdn), gu, dn)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gh.to_bits(gu), packed_layout(wgu, I, H, True))
    np.testing.assert_array_equal(gh.to_bits(dn), packed_layout(wdn, H, I, False))


PACKED = {
    # K >= 256 in both projections (the ping-pong schedule), ragged N tiles in
    # both (I = 288, H = 288), a shared expert whose width is ragged too
    "pp_ragged": Workload("pp_ragged", T=700, H=288, E=4, k=2, I=288, I_s=320, rsf=1.3),
    "pipe_small": SMALL["pipe_small"],      # K = 160 in down: the interleaved schedule
    "scmoe_gamma": SMALL["scmoe_gamma"],
    "no_shared": SMALL["no_shared"],
    # three tokens: one partial half-height tile per touched expert, most
    # experts empty, the shared expert a single 3-row tile
    "tiny_pp": Workload("tiny_pp", T=3, H=256, E=8, k=2, I=256, I_s=256),
}


@pytest.mark.parametrize("variant", ["pingpong", "pipe256w8"])
@pytest.mark.parametrize("name", list(PACKED))
def test_forward_packed_experts(monkeypatch, variant, name):
    """The 256-row tiles over the tile-blocked copies give the same bits as
    over the row-major experts (only the addresses differ), and the layer
    stays parity-green against the oracle."""
    monkeypatch.setenv("MOE_GEMM_VARIANT", variant)
    wl = PACKED[name]
    inp = moe_inputs.generate(wl, seed=6)
    gh.note(f"packed {variant} {wl.label()}")
    d = gh.Device(wl, inp)
    d.canary()
    d.run()
    rows = d.result()
    d.pack()
    d.canary()
    d.run()
    tiled = d.result()
    for key in ("out", "h", "hs"):
        if key in rows:
            np.testing.assert_array_equal(tiled[key], rows[key], err_msg=key)
    gh.check_layer(wl, inp, tiled)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("variant", ["pingpong", "pipe256w8"])
@pytest.mark.parametrize("name", list(PACKED))
def test_forward_blocked_h(monkeypatch, variant, name, packed):
    """h stage-blocked between the 256-row tiles gives the same output bits
    as h in rows (the run that probes it, checked against the oracle):
    partial and half-height tiles, experts with no rows, the shared expert
    with T not a multiple of 256, either weight layout."""
    monkeypatch.setenv("MOE_GEMM_VARIANT", variant)
    wl = PACKED[name]
    inp = moe_inputs.generate(wl, seed=8)
    gh.note(f"blocked h {variant} packed={packed} {wl.label()}")
    d = gh.Device(wl, inp)
    if packed:
        d.pack()
    d.canary()
    d.run()
    rows = d.result()
    gh.check_layer(wl, inp, rows)
    d.unprobe_h()
    d.canary()
    d.run()
    blk = d.result()
    for key in ("out", "ids", "offsets", "sorted_token", "inv_pos"):
        np.testing.assert_array_equal(blk[key], rows[key], err_msg=key)


def test_forward_graph_replay_blocked_layouts(monkeypatch):
    """A forward on the 256-row tiles with the tile-blocked copies and h
    stage-blocked, captured into a HIP graph, replays to the eager result bit
    for bit, several times with eager work in between."""
    monkeypatch.setenv("MOE_GEMM_VARIANT", "pingpong")
    torch, moe = gh.torch_and_lib()
    wl = PACKED["pp_ragged"]
    gh.note(f"graph replay, blocked layouts {wl.label()}")
    d = gh.Device(wl, moe_inputs.generate(wl, seed=9))
    d.pack()
    d.unprobe_h()
    d.run()
    eager = gh.to_bits(d.out).copy()
    out_g = torch.empty_like(d.out)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_forward(d.params, d.x, d.x_cur, d.weights, out_g, None, d.ws)  # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        moe.moe_forward(d.params, d.x, d.x_cur, d.weights, out_g, None, d.ws)
    for rep in range(3):
        out_g.fill_(0x7FC0)
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gh.to_bits(out_g), eager, err_msg=f"replay {rep}")
        d.run()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gh.to_bits(d.out), eager)


def test_forward_prefill_packed_full():
    """The measured prefill workload with the tile-blocked expert copies and
    with h stage-blocked (the bench's configuration): every output bit equal
    to the row-major run, a sample of tokens against the oracle."""
    wl = moe_inputs.WORKLOADS["prefill"]
    gh.note(f"generating {wl.label()}")
    inp = moe_inputs.generate(wl, seed=0)
    d = gh.Device(wl, inp)
    d.run()
    rows = d.result()
    d.pack()
    d.canary()
    d.run()
    tiled = d.result()
    np.testing.assert_array_equal(tiled["out"], rows["out"])
    np.testing.assert_array_equal(tiled["h"], rows["h"])
    sample = np.sort(np.random.default_rng(7).choice(wl.T, size=64, replace=False))
    gh.note(f"  {gh.check_layer(wl, inp, tiled, sample)}")
    d.unprobe_h()
    d.canary()
    d.run()
    np.testing.assert_array_equal(d.result()["out"], rows["out"])


# ------------------------------------------------ W4A16 routed experts ----

W4 = {
    # one whole 512-column stage in gate_up (H = 512); down K = 384: a
    # partial stage of three 128-column groups; shared expert beside routing
    "w4_small": Workload("w4_small", T=40, H=512, E=16, k=4, I=384, I_s=256, w4=True),
    # H = 640: a whole stage then a one-group stage; no shared expert;
    # several 16-row m-tiles per expert
    "w4_multi": Workload("w4_multi", T=96, H=640, E=8, k=2, I=256, I_s=0, rsf=1.5, w4=True),
    # clamp stress with W4 codes (large scales)
    "w4_clamp": Workload("w4_clamp", T=32, H=256, E=8, k=2, I=128, I_s=128, weight_std=0.3,
                         w4=True),
    # every E4M3 scale byte but the NaNs (both signs, zeros, subnormals, 448)
    "w4_full_range": Workload("w4_full_range", T=40, H=512, E=16, k=4, I=384, I_s=256, w4=True,
                              w4_scales="full"),
}


@pytest.mark.parametrize("name", list(W4))
def test_forward_w4(name):
    wl = W4[name]
    inp = moe_inputs.generate(wl, seed=4)
    rep, _, _ = run_and_check(wl, inp)
    assert rep["rows_checked"] == wl.T


@pytest.mark.parametrize("variant", ["pingpong", "tile128", "pipe256w8"])
@pytest.mark.parametrize("name", ["w4_small", "w4_multi", "w4_clamp"])
def test_forward_w4_tile_variant(monkeypatch, variant, name):
    """W4A16 layers on the tiled variants, forced on decode-sized batches:
    the ping-pong tile unpacks the codes itself (mostly empty 256-row tiles,
    one or two n-tiles), the others read the experts dequantised in the
    workspace."""
    monkeypatch.setenv("MOE_GEMM_VARIANT", variant)
    wl = W4[name]
    rep, _, _ = run_and_check(wl, moe_inputs.generate(wl, seed=4))
    assert rep["rows_checked"] == wl.T


def test_forward_decode_w4_full():
    rep = _full("decode_w4", None)
    assert rep["rows_checked"] == 32


@pytest.mark.parametrize("scales", ["typical", "full"])
def test_forward_prefill_w4_full(scales):
    # T * k = 65 536 rows over 64 experts: the experts expanded exactly to
    # bf16, the tensor scales on the fp32 sums, against the oracle's exact
    # weights; the measured scale draw on every token, every E4M3 scale byte
    # on a token sample
    wl = moe_inputs.WORKLOADS["prefill_w4"].with_(w4_scales=scales)
    gh.note(f"generating {wl.label()} scales={scales}")
    inp = moe_inputs.generate(wl, seed=0)
    rows = None
    if scales == "full":
        rows = np.sort(np.random.default_rng(7).choice(wl.T, size=256, replace=False))
    rep, gpu, dev = run_and_check(wl, inp, rows)
    assert rep["experts_touched"] == 64
    # without h probes and with the shared expert's tile-blocked copies (as
    # the bench runs it): the same output bits
    dev.unprobe_h()
    dev.pack()
    dev.canary()
    dev.run()
    np.testing.assert_array_equal(dev.result()["out"], gpu["out"])
    del dev


# ------------------------------------------------ finish (residual add) ----

FINISH = {
    # plain layer, the ScMoE-style residual/BDA (coefficients 1)
    "plain_bda": (Workload("fin_plain", T=96, H=256, E=16, k=3, I=128, I_s=128),
                  dict(out_scale=1.0, residual_scale=1.0)),
    # plain layer with the sandwich post-norm and a depth-scaled add
    "sandwich_scaled": (Workload("fin_sandwich", T=150, H=384, E=24, k=4, I=192, I_s=256,
                                 gamma_jitter=0.1),
                        dict(out_scale=0.6, residual_scale=0.8, post_norm=True)),
    # ScMoE pairing, residual added in place (out is the residual buffer)
    "scmoe_in_place": (Workload("fin_scmoe", T=120, H=384, E=32, k=4, I=192, I_s=256,
                                scmoe=True, gamma_jitter=0.1),
                       dict(out_scale=1.0, residual_scale=1.0, in_place=True)),
    # decode-sized (weight streaming, shared expert beside routing)
    "decode_small": (Workload("fin_decode", T=20, H=512, E=40, k=4, I=176, I_s=352),
                     dict(out_scale=2 ** -0.5, residual_scale=2 ** -0.5)),
}


@pytest.mark.parametrize("name", list(FINISH))
def test_forward_finish(name):
    """moe_forward_finish against the oracle with S8, and the fused finish
    bit for bit against the finish of the GPU's own unfinished output."""
    wl, fin = FINISH[name]
    inp = moe_inputs.generate(wl, seed=6)
    if fin.get("post_norm") and inp.get("gamma_post") is None:
        inp["gamma_post"] = (1 + 0.1 * np.random.default_rng(7).uniform(-1, 1, wl.H)).astype(np.float32)
    res_bits = moe_inputs.f32_to_bf16_bits(
        np.random.default_rng(8).standard_normal((wl.T, wl.H)).astype(np.float32) * 2)
    fin = dict(fin, residual=res_bits)
    gh.note(f"forward_finish {name} {wl.label()} {dict((k, v) for k, v in fin.items() if k != 'residual')}")
    d = gh.Device(wl, inp, finish=fin)
    d.canary()
    d.run()
    gpu = d.result()
    rep = gh.check_layer(wl, inp, gpu, finish=fin)
    gh.note(f"  {rep}")
    # the unfinished output of the same layer on the GPU: a finish that keeps
    # o (scales 1 and 0, zero residual, the same post-norm setting)
    keep = dict(residual=np.zeros_like(res_bits), out_scale=1.0, residual_scale=0.0,
                post_norm=fin.get("post_norm", False))
    d0 = gh.Device(wl, inp, finish=keep)
    d0.run()
    o = d0.result()["out"]
    want = mo.finish(o, res_bits, fin["out_scale"], fin["residual_scale"])
    got = gpu["out"]
    # values, so that -0 and +0 (from o + 0 in the keeping finish) compare equal
    assert np.array_equal(mo.bf16_to_f64(got), mo.bf16_to_f64(want)), \
        f"fused finish differs in {int(np.sum(mo.bf16_to_f64(got) != mo.bf16_to_f64(want)))} elements"


def test_forward_prefill_finish_full_sampled():
    """The prefill workload with the residual add fused into the combine
    (coefficients 1), as the bench's --finish runs it, on a token sample."""
    wl = moe_inputs.WORKLOADS["prefill"]
    inp = moe_inputs.generate(wl, seed=0)
    res_bits = moe_inputs.f32_to_bf16_bits(
        np.random.default_rng(1).standard_normal((wl.T, wl.H)).astype(np.float32))
    fin = dict(residual=res_bits, out_scale=1.0, residual_scale=1.0)
    rows = np.sort(np.random.default_rng(7).choice(wl.T, size=64, replace=False))
    gh.note(f"forward_finish {wl.label()} sampled")
    d = gh.Device(wl, inp, finish=fin)
    d.canary()
    d.run()
    rep = gh.check_layer(wl, inp, d.result(), rows, finish=fin)
    gh.note(f"  {rep}")
    assert rep["rows_checked"] == 64


# ------------------------------- W4A16 experts beyond weight streaming ----

W4_TILED = {
    # ~300 rows per expert: the LDS-tiled GEMM on the dequantised experts
    "w4_tiled": Workload("w4_tiled", T=600, H=256, E=4, k=2, I=256, I_s=128, w4=True),
    # ~2400 rows per expert, but I = 128: the W4A16 ping-pong tile needs
    # K >= 256 in both projections, so the experts are dequantised and run
    # through the bf16 tiles (down, K = 128, in the interleaved schedule)
    "w4_prefill_k128": Workload("w4_prefill_k128", T=2400, H=384, E=4, k=2, I=128, I_s=0,
                                w4=True),
    # the W4A16 ping-pong tile at its shortest K: down K = 256, two code
    # groups per tile (every step is one of a tile's first or last four);
    # N = 384 (a half-empty last column tile); no shared expert
    "w4_pingpong_k256": Workload("w4_pingpong_k256", T=2400, H=384, E=4, k=2, I=256, I_s=0,
                                 w4=True),
    # 4096 rows per expert: two or more tiles per workgroup in both
    # projections (the stage stream runs across tiles), shared expert after
    "w4_pingpong_multi": Workload("w4_pingpong_multi", T=8192, H=512, E=8, k=4, I=512, I_s=256,
                                  w4=True),
}


def _bf16_experts(inp):
    """The same layer with its W4A16 weights stored as bf16 (exactly: the
    tensor scales are powers of two here), as bf16 expert arrays."""
    ref = {k: v for k, v in inp.items()
           if not k.endswith("_q") and not k.endswith("_scale") and not k.endswith("_tscale")}
    for name in ("w_gate_up", "w_down"):
        q, sc, ts = inp[name + "_q"], inp[name + "_scale"], inp[name + "_tscale"]
        vals = [mo.dequant_w4(q[e], sc[e], ts[e]) for e in range(q.shape[0])]
        assert all(np.array_equal(mo.bf16_to_f64(mo.bf16_round(v)), v) for v in vals)
        ref[name] = np.stack([mo.bf16_round(v) for v in vals])
    return ref


@pytest.mark.parametrize("name", list(W4_TILED))
def test_forward_w4_tiled(name):
    """Prefill-sized W4A16 batches: parity with the oracle's exact
    dequantised layer, and bit-for-bit equality with the bf16 path run on
    the same weights (power-of-two tensor scales make them bf16 values, and
    scaling an fp32 sum by a power of two commutes with its roundings)."""
    wl = W4_TILED[name]
    inp = moe_inputs.generate(wl, seed=5)
    rng = np.random.default_rng(9)
    for n in ("w_gate_up_tscale", "w_down_tscale"):
        inp[n] = np.ldexp(1.0, rng.integers(-10, -7, size=wl.E)).astype(np.float32)
    rep, gpu, dw = run_and_check(wl, inp)
    ref_inp = _bf16_experts(inp)
    wl_bf16 = wl.with_(w4=False)
    gh.note(f"forward {name} as bf16 on host-rounded weights")
    d = gh.Device(wl_bf16, ref_inp)
    d.canary()
    d.run()
    g2 = d.result()
    assert np.array_equal(gpu["ids"], g2["ids"])
    assert np.array_equal(gpu["out"], g2["out"]), \
        f"differs from the bf16 path in {int(np.sum(gpu['out'] != g2['out']))} elements"
    # without h probes (as the bench runs it), then also with the shared
    # expert's tile-blocked copies: the same output bits
    dw.unprobe_h()
    dw.canary()
    dw.run()
    np.testing.assert_array_equal(dw.result()["out"], gpu["out"])
    if wl.I_s:
        dw.pack()
        dw.canary()
        dw.run()
        np.testing.assert_array_equal(dw.result()["out"], gpu["out"])
