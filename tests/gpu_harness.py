"""Helpers of the GPU parity tests: upload seeded inputs, run the library
through its C ABI, and compare with the oracle.

Parity bar (the layer's tolerances):
  * router logits within the fp32 forward-error bound of an H-term sum,
    H * 2^-24 * sum_i |x_i W_r[e,i]| (products are exact; only the order and
    rounding of the sums differ from the float64 oracle);
  * the top-k decision, given the GPU's own fp32 logits, bit-exact: ids equal
    the oracle's selection applied to those logits, and weights equal
    fp32(rsf * sigmoid(l)) within SIG_ULP ulp;
  * expert ids bit-exact against the oracle's own logits, except tokens whose
    k-th and (k+1)-th biased scores lie within 1e-5 of each other (count
    reported); for such tokens the oracle re-derives the rest of the layer
    from the GPU's ids, since either selection is correct;
  * emitted weights within the logit bound carried through the sigmoid
    (|d sigma/dl| <= 1/4) plus SIG_ULP ulp of the oracle's weight;
  * offsets, sorted_token and inv_pos bit-exact (against the oracle's
    permutation of the GPU's ids);
  * the SwiGLU outputs h (routed and shared, read through the forward's
    probes) equal the oracle's bf16 rounding, except elements where another
    rounding is as correct: the GPU's value must be a rounding of a value
    within the fp32 error bound of the exact one (K u sum|x w| for each
    K-term dot product carried through the SwiGLU, plus 2^-19 |h| for its
    exp and reciprocal), and at most 1 % of the elements may differ (count
    reported);
  * outputs |gpu - oracle| <= 2e-2 * max(1, |oracle|) elementwise, the
    oracle re-deriving y, ys and the output from the GPU's validated h (as
    for near-tie ids); the distance to the oracle's own rounding of h is
    reported beside it.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import moe_oracle as mo

NEAR_TIE = 1e-5
OUT_TOL = 2e-2
SIG_ULP = 1
U32 = 2.0 ** -24


def torch_and_lib():
    import torch
    import mixture_experts_layer_steered_amd as moe
    return torch, moe


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def dev_f32(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def to_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class Device:
    """Inputs of one workload resident on the GPU plus the output buffers.
    `finish` (optional): dict(residual=bf16 bits [T, H], out_scale,
    residual_scale, post_norm, in_place) -- the layer then runs through
    moe_forward_finish; with in_place the output overwrites the residual's
    device buffer."""

    def __init__(self, wl, inp: dict, finish: dict | None = None):
        torch, moe = torch_and_lib()
        self.torch, self.moe, self.wl, self.inp = torch, moe, wl, inp
        T, H, E, k = inp["x"].shape[0], wl.H, wl.E, wl.k
        self.T = T
        self.params = moe.make_params(T, H, E, k, wl.I, wl.I_s, wl.rsf, wl.limit, wl.scmoe, wl.eps,
                                      w4="w_gate_up_q" in inp)
        self.x = dev_bf16(torch, inp["x"])
        self.x_cur = dev_bf16(torch, inp["x_cur"]) if wl.scmoe else None
        self.w_router = dev_f32(torch, inp["w_router"])
        self.corr_bias = dev_f32(torch, inp["corr_bias"]) if inp.get("corr_bias") is not None else None
        w4 = "w_gate_up_q" in inp
        self.w_gate_up = None if w4 else dev_bf16(torch, inp["w_gate_up"])
        self.w_down = None if w4 else dev_bf16(torch, inp["w_down"])
        self.w4 = {}
        if w4:   # codes and E4M3 scale bytes; fp32 tensor scales when given
            for n in ("w_gate_up_q", "w_down_q", "w_gate_up_scale", "w_down_scale"):
                self.w4[n] = torch.from_numpy(np.ascontiguousarray(inp[n])).to("cuda")
            for n in ("w_gate_up_tscale", "w_down_tscale"):
                if inp.get(n) is not None:
                    self.w4[n] = dev_f32(torch, inp[n])
        self.ws_gate_up = dev_bf16(torch, inp["ws_gate_up"]) if wl.I_s else None
        self.ws_down = dev_bf16(torch, inp["ws_down"]) if wl.I_s else None
        self.gamma_pre = dev_f32(torch, inp["gamma_pre"]) if inp.get("gamma_pre") is not None else None
        self.gamma_post = dev_f32(torch, inp["gamma_post"]) if inp.get("gamma_post") is not None else None
        self.weights = moe.make_weights(self.w_router, self.corr_bias, self.w_gate_up, self.w_down,
                                        self.ws_gate_up, self.ws_down, self.gamma_pre,
                                        self.gamma_post, **self.w4)
        nbytes = moe.moe_workspace_size(self.params)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        self.out = torch.empty((T, H), dtype=torch.int16, device="cuda")
        self.fin = None
        self.in_place = False
        if finish is not None:
            self.residual = dev_bf16(torch, finish["residual"])
            self.fin = moe.make_finish(self.residual, finish.get("out_scale", 1.0),
                                       finish.get("residual_scale", 1.0),
                                       finish.get("post_norm", False))
            self.in_place = bool(finish.get("in_place", False))
            if self.in_place:
                self.out = self.residual
        N = T * k
        self.ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        self.w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        self.sorted_token = torch.empty(max(N, 1), dtype=torch.int32, device="cuda")
        self.inv_pos = torch.empty(max(N, 1), dtype=torch.int32, device="cuda")
        self.xr = torch.empty((T, H), dtype=torch.int16, device="cuda") if wl.scmoe else None
        self.logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        self.h = torch.empty((max(N, 1), wl.I), dtype=torch.int16, device="cuda")
        self.hs = (torch.empty((T, wl.I_s), dtype=torch.int16, device="cuda")
                   if wl.I_s else None)
        self.probes = moe.make_probes(self.ids, self.w, self.offsets, self.sorted_token,
                                      self.inv_pos, self.xr, self.logits, h=self.h,
                                      h_shared=self.hs)

    def pack(self) -> None:
        """Write the tile-blocked copies of the bf16 experts (the routed ones
        unless they are W4A16, and the shared expert with E = 1, I = I_shared)
        and hand them to the layer."""
        torch, moe, wl = self.torch, self.moe, self.wl
        extra = {}
        if not self.w4:  # W4A16 routed experts: the shared expert's copies only
            gu_n, dn_n = moe.moe_packed_experts_size(self.params)
            self.gu_packed = torch.full((gu_n,), 0x7FC0, dtype=torch.int16, device="cuda")
            self.dn_packed = torch.full((dn_n,), 0x7FC0, dtype=torch.int16, device="cuda")
            moe.moe_pack_experts(self.params, self.w_gate_up, self.w_down, self.gu_packed,
                                 self.dn_packed)
            extra = dict(w_gate_up_packed=self.gu_packed, w_down_packed=self.dn_packed)
        if wl.I_s:
            ps = moe.make_params(self.T, wl.H, 1, 1, wl.I_s, 0, wl.rsf, wl.limit, False, wl.eps)
            sgu_n, sdn_n = moe.moe_packed_experts_size(ps)
            self.sgu_packed = torch.full((sgu_n,), 0x7FC0, dtype=torch.int16, device="cuda")
            self.sdn_packed = torch.full((sdn_n,), 0x7FC0, dtype=torch.int16, device="cuda")
            moe.moe_pack_experts(ps, self.ws_gate_up, self.ws_down, self.sgu_packed,
                                 self.sdn_packed)
            extra.update(ws_gate_up_packed=self.sgu_packed, ws_down_packed=self.sdn_packed)
        self.weights = moe.make_weights(self.w_router, self.corr_bias, self.w_gate_up,
                                        self.w_down, self.ws_gate_up, self.ws_down,
                                        self.gamma_pre, self.gamma_post, **self.w4, **extra)

    def unprobe_h(self) -> None:
        """Probe everything but h and h_shared: the forward then hands h from
        gate_up to down in its own layout (stage-blocked within each 256-row
        tile on those tiles)."""
        self.probes = self.moe.make_probes(self.ids, self.w, self.offsets, self.sorted_token,
                                           self.inv_pos, self.xr, self.logits)

    def canary(self) -> None:
        """Fill every output with NaN / out-of-range bits first, so that an
        element the kernels never write shows up."""
        if not self.in_place:
            self.out.fill_(0x7FC0)
        self.ids.fill_(-7)
        self.w.fill_(float("nan"))
        self.offsets.fill_(-7)
        self.sorted_token.fill_(-7)
        self.inv_pos.fill_(-7)
        self.logits.fill_(float("nan"))
        if self.xr is not None:
            self.xr.fill_(0x7FC0)

    def run(self) -> None:
        if self.fin is not None:
            self.moe.moe_forward_finish(self.params, self.x, self.x_cur, self.weights, self.fin,
                                        self.out, self.probes, self.ws)
        else:
            self.moe.moe_forward(self.params, self.x, self.x_cur, self.weights, self.out,
                                 self.probes, self.ws)

    def result(self) -> dict:
        self.torch.cuda.synchronize()
        N = self.T * self.wl.k
        r = dict(out=to_bits(self.out), ids=self.ids.cpu().numpy(), w=self.w.cpu().numpy(),
                 offsets=self.offsets.cpu().numpy(),
                 sorted_token=self.sorted_token.cpu().numpy()[:N],
                 inv_pos=self.inv_pos.cpu().numpy()[:N], logits=self.logits.cpu().numpy(),
                 h=to_bits(self.h)[:N])
        if self.hs is not None:
            r["hs"] = to_bits(self.hs)
        if self.xr is not None:
            r["xr"] = to_bits(self.xr)
        return r


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return np.abs(a.astype(np.float64) - b.astype(np.float64)) / np.spacing(np.abs(b)).astype(np.float64)


def check_router(x_bits, w_router, corr_bias, k, rsf, logits_g, ids_g, w_g) -> dict:
    """Router parity (see the module docstring).  Returns a report with the
    oracle's routing under 'route'."""
    rep: dict = {}
    logits_o = mo.router_logits(x_bits, w_router)
    H = x_bits.shape[1]
    absdot = np.abs(mo.bf16_to_f64(x_bits)) @ np.abs(np.asarray(w_router, np.float64)).T
    lbound = H * U32 * absdot + 1e-30
    dl = np.abs(logits_g.astype(np.float64) - logits_o.astype(np.float64))
    ok = (dl <= lbound) | (np.isnan(logits_o) & np.isnan(logits_g))
    rep["logit_max_err_over_bound"] = float(np.nanmax(np.where(ok, dl / lbound, np.inf))) if dl.size else 0.0
    assert np.all(ok), "router logits outside the fp32 summation bound"
    # the top-k decision on the GPU's own logits: exact
    rg = mo.topk_route(logits_g, corr_bias, k, rsf)
    assert np.array_equal(ids_g, rg["ids"]), "top-k differs from the selection on the GPU's logits"
    ud = ulp_distance(w_g, rg["w"])
    rep["w_ulp_vs_gpu_logits"] = float(ud.max()) if ud.size else 0.0
    assert rep["w_ulp_vs_gpu_logits"] <= SIG_ULP, "weights differ from rsf*sigmoid(GPU logit)"
    # against the oracle's own logits: near-tie exemption for ids
    r = mo.topk_route(logits_o, corr_bias, k, rsf)
    mism = np.any(ids_g != r["ids"], axis=1)
    near = r["gap"] < NEAR_TIE
    rep["near_tie_tokens"] = int(near.sum())
    rep["id_mismatch_tokens"] = int(mism.sum())
    bad = np.nonzero(mism & ~near)[0]
    assert bad.size == 0, f"ids differ on non-near-tie tokens {bad[:10]} (gaps {r['gap'][bad[:10]]})"
    assert np.all((ids_g >= 0) & (ids_g < w_router.shape[0])), "ids out of range"
    assert np.all(np.diff(ids_g, axis=1) > 0), "ids not strictly ascending"
    ii = ids_g.astype(np.int64)
    w_ref = (np.float32(rsf) * np.take_along_axis(r["s"], ii, 1)).astype(np.float32)
    wb = abs(rsf) * 0.25 * np.take_along_axis(lbound, ii, 1) + SIG_ULP * np.spacing(np.abs(w_ref))
    dw = np.abs(w_g.astype(np.float64) - w_ref)
    uw = ulp_distance(w_g, w_ref)
    rep["w_max_ulp_vs_oracle"] = float(uw.max()) if dw.size else 0.0
    rep["w_beyond_4ulp"] = int(np.sum(uw > 4))   # reported: the bar is the bound below
    assert np.all(dw <= wb), "weights outside the propagated logit bound"
    rep["route"] = r
    return rep


H_FAST = 2.0 ** -19   # relative error allowed for the SwiGLU's exp and reciprocal


H_FLIP_SHARE = 1e-2   # at most this share of h elements may differ from the oracle's rounding


def validate_h(h_gpu: np.ndarray, h_ora: np.ndarray, pre_fn, limit: float, K: int) -> dict:
    """The GPU's bf16 h against the oracle's rounding (both bit patterns of
    one [n, I] block).  An element that differs must be a correct rounding of
    a value within the fp32 error bound of the exact one: |h_gpu - h| <=
    bound + half a bf16 step of h_gpu, the bound being K u sum|x w| on each
    dot product carried through the SwiGLU (|silu'| <= 1.1) plus H_FAST |h|
    (near a rounding midpoint that allows the other neighbour; where the
    dot products cancel, several steps).  And the share of differing
    elements must stay below H_FLIP_SHARE (or 16 elements): a systematic
    defect (a K stage lost, a wrong row) moves most elements by a step or
    more.  pre_fn(rows,
    cols) returns the oracle's swiglu_pre for those rows and columns.
    Returns the count and the largest (distance - half step) / bound."""
    diff = np.argwhere(h_gpu != h_ora)
    rep = {"flips": int(len(diff)), "flip_max_over_bound": 0.0}
    if len(diff) == 0:
        return rep
    assert len(diff) <= max(16, H_FLIP_SHARE * h_gpu.size), (
        f"h differs from the oracle's rounding in {len(diff)} of {h_gpu.size} elements")
    r, c = diff[:, 0], diff[:, 1]
    ur, ri = np.unique(r, return_inverse=True)
    uc, ci = np.unique(c, return_inverse=True)
    pre = pre_fn(ur, uc)
    g, u, h = pre["g"][ri, ci], pre["u"][ri, ci], pre["h"][ri, ci]
    L = float(np.float32(limit))
    gc, uc_ = np.minimum(g, L), np.clip(u, -L, L)
    silu = gc / (1.0 + np.exp(-gc))
    eps = K * U32
    bound = (1.1 * np.abs(uc_) * eps * pre["gabs"][ri, ci] + np.abs(silu) * eps * pre["uabs"][ri, ci]
             + H_FAST * np.abs(h))
    vg = mo.bf16_to_f64(h_gpu[r, c])
    half_step = np.spacing(np.abs(vg).astype(np.float32)).astype(np.float64) * 2.0 ** 15
    ratio = (np.abs(vg - h) - half_step) / np.maximum(bound, 1e-300)
    ok = np.isfinite(vg) & (ratio <= 1.0)
    rep["flip_max_over_bound"] = float(ratio.max())
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, (
        f"h differs beyond a valid rounding at {bad.size} of {len(diff)} elements, e.g. "
        f"{[(int(r[i]), int(c[i]), float(vg[i]), float(h[i]), float(bound[i])) for i in bad[:3]]}")
    return rep


def check_layer(wl, inp: dict, gpu: dict, rows: np.ndarray | None = None,
                finish: dict | None = None) -> dict:
    """Compare one GPU forward with the oracle.  `rows` = token sample for
    the output check (None = all tokens); routing and the permutation are
    always checked on every token; `finish` as in Device (the oracle then
    adds S8).  Returns a report; raises AssertionError on any violation."""
    kw = dict(k=wl.k, rsf=wl.rsf, limit=wl.limit, scmoe=wl.scmoe, eps=wl.eps)
    T = inp["x"].shape[0]
    rep: dict = {}
    # --- routing on every token (the oracle's router only: cheap)
    if wl.scmoe:
        xr = mo.rmsnorm_bf16(inp["x"], inp.get("gamma_pre"), wl.eps)
        rep["xr_mismatch"] = int(np.sum(xr != gpu["xr"]))
        assert rep["xr_mismatch"] == 0, f"pre-norm output differs in {rep['xr_mismatch']} elements"
    else:
        xr = inp["x"]
    rrep = check_router(xr, inp["w_router"], inp.get("corr_bias"), wl.k, wl.rsf,
                        gpu["logits"], gpu["ids"], gpu["w"])
    rrep.pop("route")
    rep.update(rrep)
    ids_g = gpu["ids"]
    # --- permutation of the GPU's ids, bit-exact
    p = mo.permute(ids_g, wl.E)
    for key in ("offsets", "sorted_token", "inv_pos"):
        assert np.array_equal(gpu[key], p[key]), f"{key} differs"
    rep["experts_touched"] = int(np.sum(p["counts"] > 0))
    rep["max_over_mean_count"] = float(p["counts"].max() / max(p["counts"].mean(), 1e-9))
    # --- outputs
    if rows is None:
        rows = np.arange(T)
    sub = mo.take_rows(inp, rows)
    if finish is not None:
        kw.update(post_norm=bool(finish.get("post_norm", False)),
                  residual=np.asarray(finish["residual"])[rows],
                  out_scale=finish.get("out_scale", 1.0),
                  residual_scale=finish.get("residual_scale", 1.0))
    ids_sub = ids_g[rows]
    res = mo.forward(sub, ids=ids_sub, **kw)
    o_gpu = mo.bf16_to_f64(gpu["out"][rows])
    assert np.all(np.isfinite(o_gpu)), "non-finite output (unwritten element?)"
    o_own = mo.bf16_to_f64(res["out"])
    d_own = np.abs(o_gpu - o_own) / (OUT_TOL * np.maximum(1.0, np.abs(o_own)))
    rep["out_max_d_over_tol_oracle_h"] = float(d_own.max()) if d_own.size else 0.0
    given = {}
    if "h" in gpu:
        # the GPU's h rows in the oracle's permuted order for the checked tokens
        k = wl.k
        ps = mo.permute(ids_sub, wl.E)
        src = gpu["inv_pos"].reshape(T, k)[rows].reshape(-1)       # GPU row of (token, slot)
        h_sub = np.empty((len(rows) * k, wl.I), dtype=np.uint16)
        h_sub[ps["inv_pos"]] = gpu["h"][src]
        h_ora = mo.bf16_round(res["h_perm"])
        xr_sub = res["xr"]
        offs = ps["offsets"]

        def pre_routed(prow, cols):
            out = {n: np.zeros((len(prow), len(cols))) for n in ("g", "u", "h", "gabs", "uabs")}
            e_of = np.searchsorted(offs, prow, side="right") - 1
            for e in np.unique(e_of):
                sel = np.nonzero(e_of == e)[0]
                a = mo.bf16_to_f64(xr_sub[ps["sorted_token"][prow[sel]]])
                pe = mo.swiglu_pre(a, mo.expert_weights(inp, int(e))[0], wl.limit, cols)
                for n in out:
                    out[n][sel] = pe[n]
            return out

        hv = validate_h(h_sub, h_ora, pre_routed, wl.limit, wl.H)
        rep["h_flips"], rep["h_flip_max_over_bound"] = hv["flips"], hv["flip_max_over_bound"]
        given["h_given"] = mo.bf16_to_f64(h_sub)
        if "hs" in gpu and res.get("hs") is not None:
            hs_sub = gpu["hs"][rows]
            x_sh = sub["x_cur"] if wl.scmoe else sub["x"]

            def pre_shared(prow, cols):
                return mo.swiglu_pre(mo.bf16_to_f64(x_sh[prow]), inp["ws_gate_up"], wl.limit, cols)

            hv = validate_h(hs_sub, mo.bf16_round(res["hs"]), pre_shared, wl.limit, wl.H)
            rep["hs_flips"] = hv["flips"]
            rep["hs_flip_max_over_bound"] = hv["flip_max_over_bound"]
            given["hs_given"] = mo.bf16_to_f64(hs_sub)
        if rep["h_flips"] or rep.get("hs_flips"):
            res = mo.forward(sub, ids=ids_sub, **kw, **given)
    o_ref = mo.bf16_to_f64(res["out"])
    d = np.abs(o_gpu - o_ref) / (OUT_TOL * np.maximum(1.0, np.abs(o_ref)))
    rep["out_max_d_over_tol"] = float(d.max()) if d.size else 0.0
    rep["out_exact_frac"] = float(np.mean(o_gpu == o_ref)) if d.size else 1.0
    rep["rows_checked"] = int(len(rows))
    assert rep["out_max_d_over_tol"] <= 1.0, f"output tolerance exceeded: {rep}"
    return rep
