"""Seeded synthetic inputs for the routed-MoE MLP forward.

This module is the only code that the CPU oracle and the HIP library's
callers (tests, bench.py, the smoke entry) both use.  It draws random
tensors and stores them in the layouts the layer consumes; it holds none
of the layer's arithmetic (no router, no top-k, no SwiGLU, no combine).

Workloads (sizes and value distributions are those the layer is measured
on; there is no public dataset or benchmark for this path, so every input
is synthetic):

  tiny     T=64    H=128  E=8   k=2 I=256  I_s=256  rsf=1.0 L=7.0
  decode   T=32    H=4096 E=64  k=8 I=1408 I_s=2816 rsf=1.0 L=7.0
  prefill  T=8192  H=4096 E=64  k=8 I=1536 I_s=1536 rsf=1.0 L=7.0
  zipf     T=16384 H=6144 E=256 k=8 I=2048 I_s=2048 rsf=2.5 L=7.0,
           router rows scaled by a Zipf(s=1.1) law over a seeded
           permutation of the expert ids (RMS-preserving, see below)
  scmoe    T=8192  H=4096 E=128 k=8 I=1024 I_s=2048 rsf=1.0 L=7.0,
           two inputs (preceding-layer and current hidden), RMSNorm
           eps 1e-6 before routing and after the merge
  decode_w4  the decode shape with W4A16 routed experts (below)
  prefill_w4 the prefill shape with W4A16 routed experts

Distributions: activations bf16 N(0,1); expert and shared weights bf16
N(0,0.02); router weights fp32 N(0,0.02); correction bias fp32
U(-0.1,0.1); RMSNorm gains 1 (or 1+U(-j,j) when a jitter j is asked).
bf16 tensors are held as uint16 bit patterns (round-to-nearest-even of
the fp32 draw).

W4A16 routed experts (workloads with w4): per weight a uniform nibble u in
[0, 15] (the value is u - 8; 4-byte words of 8 columns, byte j holding
columns j and j + 4 in its low and high nibble); per row and group of 128
columns a one-byte OCP E4M3 scale code, stored [K/128, rows]; per expert and
projection an fp32 tensor scale.  Scale codes: "typical" draws a positive
code with exponent field 6, 7 or 8 and any mantissa (values 1/2 .. 3.75,
RMS about 1.94), and the tensor scale weight_std / (sqrt(21.5) * 1.94) *
U(0.8, 1.25) (21.5 is the mean of (u - 8)^2), so the weights have about the
bf16 experts' spread; "full" draws every code except the two NaN patterns
uniformly (both signs, zeros, subnormals, up to 448), with tensor scale
weight_std / (sqrt(21.5) * 100) * U(0.8, 1.25).  The shared expert stays
bf16.

Random streams: numpy PCG64 children of SeedSequence(seed), spawned in a
fixed order: x (x_prev for ScMoE), x_cur, W_r, b, W_gu[e] for e=0..E-1,
W_d[e] for e=0..E-1, W_s_gu, W_s_d, gamma, Zipf permutation.  Each
expert draws from its own stream, so experts are generated in parallel
threads and one expert can be regenerated alone.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

WEIGHT_STD = 0.02
BIAS_RANGE = 0.1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    I_s: int
    rsf: float = 1.0
    limit: float = 7.0
    scmoe: bool = False
    eps: float = 1e-6
    zipf_s: float = 0.0      # 0 = router rows unscaled
    weight_std: float = WEIGHT_STD
    gamma_jitter: float = 0.0
    w4: bool = False         # routed experts in W4A16 form
    w4_scales: str = "typical"  # W4A16 scale codes: "typical" or "full" (every E4M3 code)

    def label(self) -> str:
        s = (f"{self.name}_T{self.T}_H{self.H}_E{self.E}_k{self.k}"
             f"_I{self.I}_Is{self.I_s}")
        return s

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", T=64, H=128, E=8, k=2, I=256, I_s=256),
    "decode": Workload("decode", T=32, H=4096, E=64, k=8, I=1408, I_s=2816),
    "prefill": Workload("prefill", T=8192, H=4096, E=64, k=8, I=1536, I_s=1536),
    "zipf": Workload("zipf", T=16384, H=6144, E=256, k=8, I=2048, I_s=2048,
                     rsf=2.5, zipf_s=1.1),
    "scmoe": Workload("scmoe", T=8192, H=4096, E=128, k=8, I=1024, I_s=2048,
                      scmoe=True, eps=1e-6),
    "decode_w4": Workload("decode_w4", T=32, H=4096, E=64, k=8, I=1408, I_s=2816, w4=True),
    "prefill_w4": Workload("prefill_w4", T=8192, H=4096, E=64, k=8, I=1536, I_s=1536, w4=True),
}

W4_GROUP = 128
W4_CODE_RMS = float(np.sqrt(21.5))  # RMS of u - 8 over uniform u in [0, 15]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (round to nearest even, NaN kept quiet).

    Used only to store the drawn inputs; the oracle and the kernels carry
    their own conversions.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + (((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF))) >> np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def _normal_bf16(seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seq))
    v = g.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v).reshape(shape)


# the RMS of the scale values each draw gives, for the tensor scale that
# puts the weights at about weight_std (a property of the code sets below)
W4_SCALE_RMS = {"typical": 1.94, "full": 100.0}


def _w4_matrix(g: np.random.Generator, R: int, K: int, std: float,
               scales: str) -> tuple[np.ndarray, np.ndarray, np.float32]:
    """One W4A16 matrix [R, K]: packed nibbles uint8 [R, K/2], E4M3 scale
    codes uint8 [K/128, R] and its fp32 tensor scale."""
    q = g.integers(0, 256, size=(R, K // 2), dtype=np.uint8)
    groups = (K + W4_GROUP - 1) // W4_GROUP
    if scales == "typical":
        field = g.integers(6, 9, size=(groups, R))
        mant = g.integers(0, 8, size=(groups, R))
        sc = ((field << 3) | mant).astype(np.uint8)
    elif scales == "full":
        # every byte but the NaN patterns 0x7F and 0xFF
        sc = g.integers(0, 254, size=(groups, R)).astype(np.uint8)
        sc = np.where(sc >= 0x7F, sc + 1, sc).astype(np.uint8)
    else:
        raise ValueError(f"w4_scales {scales!r}")
    ts = np.float32(std / (W4_CODE_RMS * W4_SCALE_RMS[scales]) * g.uniform(0.8, 1.25))
    return q, sc, ts


def zipf_row_scales(E: int, s: float, perm: np.ndarray) -> np.ndarray:
    """Per-expert router-row scales (pi(e)+1)^-s * sqrt(E / sum_j (j+1)^-2s).

    The second factor keeps the matrix RMS equal to the unscaled draw's,
    so only the spread of row norms changes.
    """
    ranks = np.arange(1, E + 1, dtype=np.float64)
    norm = np.sqrt(E / np.sum(ranks ** (-2.0 * s)))
    return ((perm.astype(np.float64) + 1.0) ** (-s) * norm).astype(np.float32)


def generate(w: Workload, seed: int = 0, *, T: int | None = None,
             experts: bool = True) -> dict:
    """Draw every input of workload `w`.

    Returns a dict of numpy arrays:
      x            uint16 [T,H]   (x_prev for ScMoE: the routed input)
      x_cur        uint16 [T,H]   (ScMoE only: the shared expert's input)
      w_router     float32 [E,H]
      corr_bias    float32 [E]
      w_gate_up    uint16 [E,2I,H]  gate rows [0,I), up rows [I,2I)
      w_down       uint16 [E,H,I]
        or, with w4: w_gate_up_q uint8 [E,2I,H/2], w_gate_up_scale uint8
        (E4M3) [E,H/128,2I], w_gate_up_tscale float32 [E], w_down_q uint8
        [E,H,I/2], w_down_scale uint8 [E,I/128,H], w_down_tscale float32 [E]
      ws_gate_up   uint16 [2I_s,H]  (absent when I_s == 0)
      ws_down      uint16 [H,I_s]
      gamma_pre    float32 [H]   (ScMoE only)
      gamma_post   float32 [H]   (ScMoE only)
    `T` overrides the token count (the first rows of the same stream are
    kept only when the same T is used; a different T is a different draw).
    `experts=False` skips the routed expert weights (router-only checks).
    """
    T = w.T if T is None else T
    H, E, I, I_s = w.H, w.E, w.I, w.I_s
    kids = np.random.SeedSequence(seed).spawn(4 + 2 * E + 4)
    k_x, k_xc, k_wr, k_b = kids[0:4]
    k_gu = kids[4:4 + E]
    k_d = kids[4 + E:4 + 2 * E]
    k_sgu, k_sd, k_gamma, k_perm = kids[4 + 2 * E:4 + 2 * E + 4]

    out: dict = {}
    out["x"] = _normal_bf16(k_x, (T, H), 1.0)
    if w.scmoe:
        out["x_cur"] = _normal_bf16(k_xc, (T, H), 1.0)

    g = np.random.Generator(np.random.PCG64(k_wr))
    wr = g.standard_normal(E * H, dtype=np.float32).reshape(E, H)
    wr *= np.float32(w.weight_std)
    if w.zipf_s > 0.0:
        perm = np.random.Generator(np.random.PCG64(k_perm)).permutation(E)
        wr *= zipf_row_scales(E, w.zipf_s, perm)[:, None]
    out["w_router"] = wr

    g = np.random.Generator(np.random.PCG64(k_b))
    out["corr_bias"] = g.uniform(-BIAS_RANGE, BIAS_RANGE, E).astype(np.float32)

    if experts and w.w4:
        gq = np.empty((E, 2 * I, H // 2), dtype=np.uint8)
        gs = np.empty((E, (H + W4_GROUP - 1) // W4_GROUP, 2 * I), dtype=np.uint8)
        gt = np.empty(E, dtype=np.float32)
        dq = np.empty((E, H, I // 2), dtype=np.uint8)
        ds = np.empty((E, (I + W4_GROUP - 1) // W4_GROUP, H), dtype=np.uint8)
        dt = np.empty(E, dtype=np.float32)

        def one_w4(e):
            gq[e], gs[e], gt[e] = _w4_matrix(np.random.Generator(np.random.PCG64(k_gu[e])),
                                             2 * I, H, w.weight_std, w.w4_scales)
            dq[e], ds[e], dt[e] = _w4_matrix(np.random.Generator(np.random.PCG64(k_d[e])),
                                             H, I, w.weight_std, w.w4_scales)

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one_w4, range(E)))
        out["w_gate_up_q"], out["w_gate_up_scale"], out["w_gate_up_tscale"] = gq, gs, gt
        out["w_down_q"], out["w_down_scale"], out["w_down_tscale"] = dq, ds, dt
    elif experts:
        wgu = np.empty((E, 2 * I, H), dtype=np.uint16)
        wd = np.empty((E, H, I), dtype=np.uint16)

        def one(e):
            wgu[e] = _normal_bf16(k_gu[e], (2 * I, H), w.weight_std)
            wd[e] = _normal_bf16(k_d[e], (H, I), w.weight_std)

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(E)))
        out["w_gate_up"] = wgu
        out["w_down"] = wd

    if I_s > 0:
        out["ws_gate_up"] = _normal_bf16(k_sgu, (2 * I_s, H), w.weight_std)
        out["ws_down"] = _normal_bf16(k_sd, (H, I_s), w.weight_std)

    if w.scmoe:
        g = np.random.Generator(np.random.PCG64(k_gamma))
        if w.gamma_jitter > 0.0:
            j = w.gamma_jitter
            out["gamma_pre"] = (1.0 + g.uniform(-j, j, H)).astype(np.float32)
            out["gamma_post"] = (1.0 + g.uniform(-j, j, H)).astype(np.float32)
        else:
            out["gamma_pre"] = np.ones(H, dtype=np.float32)
            out["gamma_post"] = np.ones(H, dtype=np.float32)
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening), for display and
    for feeding tensors to torch."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
