"""Small shared helpers for the tests (no layer arithmetic here)."""
import json
import os

import numpy as np

import moe_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_hand_example():
    """The hand-worked example as (inputs dict, params dict, expected dict)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        d = json.load(f)
    i = d["inputs"]
    bf = lambda v: moe_inputs.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))
    inp = dict(
        x=bf(i["x"]),
        w_router=np.asarray(i["w_router"], dtype=np.float32),
        corr_bias=np.asarray(i["corr_bias"], dtype=np.float32),
        w_gate_up=bf(i["w_gate_up"]),
        w_down=bf(i["w_down"]),
        ws_gate_up=bf(i["ws_gate_up"]),
        ws_down=bf(i["ws_down"]),
    )
    return inp, d["params"], d["expected"]


def tiny_inputs(T=6, H=8, E=5, k=2, I=4, I_s=3, seed=0, std=0.5, bias=0.1,
                router_std=0.5, scmoe=False):
    """Random small inputs with large weights so that clamps are exercised."""
    w = moe_inputs.Workload("t", T=T, H=H, E=E, k=k, I=I, I_s=I_s, scmoe=scmoe,
                            weight_std=std)
    inp = moe_inputs.generate(w, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    inp["w_router"] = (rng.standard_normal((E, H)) * router_std).astype(np.float32)
    inp["corr_bias"] = rng.uniform(-bias, bias, E).astype(np.float32)
    return inp
