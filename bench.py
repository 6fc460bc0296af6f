#!/usr/bin/env python3
"""Throughput of the routed-MoE MLP forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode] [--finish]

One step = one moe_forward call (router, top-k, permute, grouped gate_up
with the SwiGLU epilogue, grouped down, combine) over one batch of seeded
synthetic input already resident in HBM.  W untimed steps, then K timed
steps between two device synchronisations.  Prints one JSON line.

The default workload is the decode-shaped layer (T=32, H=4096, E=64,
top-8, I=1408, shared I_s=2816), which is bound by HBM bandwidth; the
prefill, zipf and scmoe workloads (bound by the bf16 matrix cores) and
decode_w4 (the decode shape with W4A16 routed experts) can be asked for
with --workload.  --finish runs moe_forward_finish instead: the residual
add after the layer output, fused into the combine.

roofline: the dominant kernel is the grouped gate_up launch.  With few
rows per expert (HBM-bound, weight streaming) it holds the routed experts
only: moe_forward runs the shared expert on a second stream beside the
routing kernels.  Otherwise routed and shared experts share the launch.
Its average duration is measured live with HIP events recorded by
moe_forward itself on its stream at the boundaries of that step, on every
8th timed step (--event-every; an event is a packet in the stream that
delays the next launch by microseconds, so the other steps run without).  Algorithmic work per launch:
  HBM-bound:  bytes = sum over touched experts of 2*I*H*2 (gate/up weights)
              + T*H*2 (x) + T*k*I*2 (h out)
  MFMA-bound: flops = 2*T*k*H*2I + 2*T*H*2I_s
traffic: FETCH_SIZE + WRITE_SIZE per launch from the committed rocprofv3
counter summary of that kernel, when it was taken on the current kernel
source (else null).

measured peaks: before the workload, two diagnostic kernels of the library
measure what this GPU delivers -- bf16 MFMA throughput (four independent
32x32x16 MFMA chains per wavefront, two workgroups of four wavefronts per
CU, varied non-zero operands) and HBM read bandwidth (a 4 GiB read stream,
non-temporal 16-byte loads) -- and the roofline record carries the
fraction against that measured peak beside the one against the published
peak (--no-probe-peaks skips them).

expert layout: the bf16 experts' tile-blocked copies (moe_pack_experts) are
written once before any timing, like a weight load, and handed to the layer
beside the row-major weights (config.expert_layout); the 256-row tiles of
prefill-sized batches read them, the other tiles the row-major weights.
--row-major-experts leaves them out.

cpu_baseline: the CPU oracle (float64 NumPy, untuned) timed on this host on
a bounded sample of the same batch, with the host's CPU model and BLAS.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE fwd tokens/s; % bf16 MFMA peak (prefill), % HBM GB/s (decode)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_MFMA_PEAK_TFLOPS = 157.3
KERNEL_SOURCES = ["grouped_gemm.hip", "kernels.h", "common.h"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_steered_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic(workload_label: str):
    path = os.path.join(ROOT, "profiles", f"gate_up_{workload_label}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream).
    They only time: created without the system-scope fence of a default
    event, whose cache writeback and invalidation at every record would
    stall the stream between the kernels being timed."""

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, ev: int) -> None:
        self.hip.hipEventDestroy(ev)


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def blas_backend() -> str:
    try:
        from threadpoolctl import threadpool_info
        b = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '?')})"
             for i in threadpool_info() if i.get("user_api") == "blas"]
        if b:
            return "; ".join(b)
    except Exception:
        pass
    return "unknown"


def measure_peaks(moe, torch) -> dict:
    """Measured bf16 MFMA throughput and HBM read bandwidth of this GPU (the
    library's probe kernels, timed with events on the stream they run on;
    the median of several launches)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    wgs, iters = 2 * cus, 40000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    moe.moe_probe_mfma_bf16(wgs, 1000, sink)
    mfma = []
    for _ in range(5):
        a, b = ev(), ev()
        a.record()
        flops = moe.moe_probe_mfma_bf16(wgs, iters, sink)
        b.record()
        torch.cuda.synchronize()
        mfma.append(flops / (a.elapsed_time(b) * 1e-3) / 1e12)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    best = None
    for per_cu in (1, 2, 4, 8):   # workgroups per CU: the best median
        rwgs = per_cu * cus
        rsink = torch.empty(rwgs * 256, dtype=torch.int32, device="cuda")
        moe.moe_probe_hbm_read(buf, nbytes, rwgs, rsink)
        hbm = []
        for _ in range(7):
            a, b = ev(), ev()
            a.record()
            moe.moe_probe_hbm_read(buf, nbytes, rwgs, rsink)
            b.record()
            torch.cuda.synchronize()
            hbm.append(nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
        hbm.sort()
        if best is None or hbm[len(hbm) // 2] > best[0]:
            best = (hbm[len(hbm) // 2], hbm[-1], rwgs)
    del buf
    mfma.sort()
    return {"mfma_bf16_tflops": round(mfma[len(mfma) // 2], 1),
            "mfma_bf16_tflops_max": round(mfma[-1], 1),
            "hbm_read_gbs": round(best[0], 1), "hbm_read_gbs_max": round(best[1], 1),
            "method": f"moe_probe_mfma_bf16: {wgs} workgroups x {iters} rounds of four "
                      f"32x32x16 bf16 MFMA chains per wavefront (median of 5); "
                      f"moe_probe_hbm_read: 4 GiB read once, each workgroup streaming one "
                      f"contiguous block in 16 KB steps of non-temporal 16-byte loads, the best "
                      f"median of 7 over 1, 2, 4 and 8 workgroups per CU ({best[2]} workgroups)"}


def cpu_baseline(wl, inp, sample_tokens: int, min_seconds: float, residual=None) -> dict:
    """The oracle, as it stands, on consecutive chunks of `sample_tokens`
    tokens of the same batch (wrapping around it), one oracle forward per
    chunk, until at least `min_seconds` of CPU time (at most 64 chunks)."""
    from oracle import moe_oracle as mo
    import numpy as np
    s = min(sample_tokens, wl.T)
    done, chunks, dt = 0, 0, 0.0
    while chunks < 64 and (dt < min_seconds or chunks == 0):
        rows = (np.arange(s) + chunks * s) % wl.T
        sub = mo.take_rows(inp, rows)
        fin = {} if residual is None else dict(residual=residual[rows])
        t0 = time.perf_counter()
        mo.forward(sub, k=wl.k, rsf=wl.rsf, limit=wl.limit, scmoe=wl.scmoe, eps=wl.eps, **fin)
        dt += time.perf_counter() - t0
        done += s
        chunks += 1
    return {"value": round(done / dt, 3), "unit": "tokens/s", "cores": cpu_threads(),
            "kind": "oracle", "cpu_model": cpu_model(), "blas": blas_backend(),
            "sample": f"{chunks} oracle forwards of {s} consecutive tokens of the same batch of "
                      f"{wl.T} ({done} tokens, {dt:.1f} s, float64 NumPy)"}


def calibrate_copy(nbytes: int, reps: int) -> None:
    """A plain streaming kernel of known size (read nbytes, write nbytes), to
    scale the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "neg_f32", "read_bytes": nbytes, "write_bytes": nbytes,
                      "reps": reps}))


# where the grouped GEMM kernels carry their gate_up flag: the third argument
# of the pipelined tiles' shape, the last of the LDS-staged tiles', the first
# of the weight-streaming tiles'
_GATEUP_FLAG = (re.compile(r"PipeShape<\d+, \d+, (true|false)"),
                re.compile(r"grouped_gemm_kernel<(?:\d+, ){4}(true|false)"),
                re.compile(r"grouped_\w+_kernel<(true|false)"))


def _grouped_kind(name: str) -> str | None:
    if "grouped_" not in name:
        return None
    for rx in _GATEUP_FLAG:
        m = rx.search(name)
        if m:
            return "gate_up" if m.group(1) == "true" else "down"
    return None


def _is_gate_up(name: str) -> bool:
    return _grouped_kind(name) == "gate_up"


def _counter_means(csv_path: str, counter: str, select, full_grid: bool = False
                   ) -> tuple[float, int]:
    """Mean of one rocprofv3 counter (CSV output) over the dispatches of the
    kernels that `select` accepts by name (with full_grid, only those with the
    largest grid among them: the routed launch, not the shared expert's
    narrower one on the second stream)."""
    import csv
    rows = [r for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and select(r["Kernel_Name"])]
    if full_grid and rows:
        g = max(int(r["Grid_Size"]) for r in rows)
        rows = [r for r in rows if int(r["Grid_Size"]) == g]
    vals = [float(r["Counter_Value"]) for r in rows]
    if not vals:
        raise SystemExit(f"no {counter} rows for the selected kernels in {csv_path}")
    return sum(vals) / len(vals), len(vals)


def write_traffic(workload: str, fetch_csv: str, write_csv: str, cal_fetch_csv: str,
                  cal_write_csv: str, command: str) -> None:
    """HBM traffic of the dominant launch from rocprofv3 counter runs:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the gate_up kernel, each
    scaled by what the same counter reads for the calibration copy (a
    torch.neg over 1 GiB: 1 GiB read, 1 GiB written).  Writes
    profiles/gate_up_<workload>_traffic.json, stamped with the kernel
    source hash so that bench.py drops it once the kernel changes."""
    import moe_inputs
    wl = moe_inputs.WORKLOADS[workload]
    f_kib, nf = _counter_means(fetch_csv, "FETCH_SIZE", _is_gate_up, full_grid=True)
    w_kib, nw = _counter_means(write_csv, "WRITE_SIZE", _is_gate_up, full_grid=True)
    cf_kib, _ = _counter_means(cal_fetch_csv, "FETCH_SIZE", lambda n: "neg" in n)
    cw_kib, _ = _counter_means(cal_write_csv, "WRITE_SIZE", lambda n: "neg" in n)
    gib = float(1 << 30)
    f_scale, w_scale = gib / (cf_kib * 1024.0), gib / (cw_kib * 1024.0)
    fetch_b = f_kib * 1024.0 * f_scale
    write_b = w_kib * 1024.0 * w_scale
    kernel = ("grouped gate_up + SwiGLU (routed experts)" if wl.T * wl.k <= 64 * wl.E
              else "grouped gate_up + SwiGLU (routed + shared, one launch)")
    out = {"workload": wl.label(), "kernel": kernel,
           "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
           "dispatches": [nf, nw],
           "copy_calibration": {"kernel": "torch.neg fp32, 1 GiB in, 1 GiB out",
                                "fetch_kib": round(cf_kib, 1), "write_kib": round(cw_kib, 1),
                                "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
           "hbm_bytes_per_launch": round(fetch_b + write_b),
           "hbm_fetch_bytes": round(fetch_b), "hbm_write_bytes": round(write_b),
           "command": command, "kernel_source_sha256": kernel_source_sha()}
    path = os.path.join(ROOT, "profiles", f"gate_up_{wl.label()}_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def write_mfma(workload: str, csv_path: str, command: str) -> None:
    """MFMA counters of the grouped GEMM launches from one rocprofv3 --pmc
    run (counters MfmaUtil, MfmaFlopsBF16, GRBM_GUI_ACTIVE): per
    projection, the mean MFMA-busy share of the SIMDs' active cycles and the
    bf16 MFMA flops the hardware executed per launch against the algorithmic
    flops (the excess is the padding of partly filled row tiles).  Writes
    profiles/mfma_<workload>.json."""
    import csv
    import moe_inputs
    wl = moe_inputs.WORKLOADS[workload]
    T, H, k, I, Is = wl.T, wl.H, wl.k, wl.I, wl.I_s
    routed = {"gate_up": 2 * T * k * H * 2 * I, "down": 2 * T * k * I * H}
    shared = {"gate_up": 2 * T * H * 2 * Is, "down": 2 * T * Is * H}
    # W4A16 routed experts run in launches of their own (grouped_pp_w4_*),
    # the bf16 shared expert in the bf16 tile's launches; otherwise one launch
    # per projection carries both
    split = wl.w4
    vals: dict = {}
    for r in csv.DictReader(open(csv_path)):
        kind = _grouped_kind(r["Kernel_Name"])
        if kind is None:
            continue
        part = ("routed" if "_w4_" in r["Kernel_Name"] else "shared") if split else "all"
        vals.setdefault((kind, part, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    out = {"workload": wl.label(), "command": command, "kernel_source_sha256": kernel_source_sha(),
           "projections": {}}
    parts = ("routed", "shared") if split else ("all",)
    for kind in ("gate_up", "down"):
        for part in parts:
            util = vals.get((kind, part, "MfmaUtil"), [])
            flops = vals.get((kind, part, "MfmaFlopsBF16"), [])
            gui = vals.get((kind, part, "GRBM_GUI_ACTIVE"), [])
            if not util:
                continue
            algo = {"routed": routed[kind], "shared": shared[kind],
                    "all": routed[kind] + shared[kind]}[part]
            mean = lambda v: sum(v) / len(v) if v else None  # noqa: E731
            f = mean(flops)
            key = kind if part == "all" else f"{kind}_{part}"
            out["projections"][key] = {
                "dispatches": len(util), "mfma_util_percent": round(mean(util), 2),
                "mfma_flops_executed_per_launch": f, "algorithmic_flops_per_launch": algo,
                "executed_over_algorithmic": round(f / algo, 4) if f else None,
                "grbm_gui_active_per_launch": mean(gui)}
    path = os.path.join(ROOT, "profiles", f"mfma_{wl.label()}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def router_backward_bench(args) -> int:
    """Gradients of the router GEMM (moe_router_backward: grad_x, grad_W,
    grad_b) on the prefill batch (T=8192, H=4096, E=64): one JSON line.
    Work per call: 2*T*E*H flops for grad_x and as many for grad_W, on the
    fp32 matrix cores."""
    import numpy as np
    import torch
    import moe_inputs
    import mixture_experts_layer_steered_amd as moe

    T, H, E = 8192, 4096, 64
    steps = args.steps if args.steps is not None else 50
    warmup = args.warmup if args.warmup is not None else 5
    rng = np.random.default_rng(0)
    x_bits = moe_inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    dl = (rng.standard_normal((T, E)) * 0.1).astype(np.float32)
    x = torch.from_numpy(x_bits.view(np.int16)).to("cuda")
    wd = torch.from_numpy(w).to("cuda")
    dld = torch.from_numpy(dl).to("cuda")
    p = moe.make_params(T, H, E, 1, 8, 0, 1.0, 7.0)
    gx = torch.empty((T, H), dtype=torch.int16, device="cuda")
    gw = torch.empty((E, H), dtype=torch.float32, device="cuda")
    gb = torch.empty((E,), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(moe.moe_router_backward_workspace_size(p), 16), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup):
        moe.moe_router_backward(p, dld, x, wd, gx, gw, gb, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        moe.moe_router_backward(p, dld, x, wd, gx, gw, gb, ws)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    ev_ms = e0.elapsed_time(e1) / steps
    flops = 4 * T * E * H
    achieved = flops / (ev_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as mo
        n, done, dt = 1024, 0, 0.0
        while dt < args.cpu_seconds and done < 64 * n:
            rows = (np.arange(n) + done) % T
            ts = time.perf_counter()
            mo.router_backward(dl[rows], x_bits[rows], w)
            dt += time.perf_counter() - ts
            done += n
        cpu = {"value": round(done / dt, 1), "unit": "tokens/s", "cores": cpu_threads(),
               "kind": "oracle", "cpu_model": cpu_model(), "blas": blas_backend(),
               "sample": f"{done // n} oracle router backwards of {n} tokens of the same batch "
                         f"({done} tokens, {dt:.1f} s, float64 NumPy)"}
    line = {
        "metric": "router backward tokens/s", "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"router_backward_T{T}_H{H}_E{E}", "T": T, "H": H, "E": E,
                   "outputs": "grad_x bf16, grad_w fp32, grad_b fp32", "parallelism": "ep1_tp1"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "router backward (grad_x and grad_W fp32 GEMMs, grad_b sum), "
                               "all launches of one call",
                     "algorithmic_flops_per_launch": flops, "avg_launch_ms": round(ev_ms, 5)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "decode_w4", "prefill", "prefill_w4", "zipf", "scmoe"])
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens the CPU oracle runs on (default: by workload)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle time to spend on the baseline sample (at least)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row-major-experts", action="store_true",
                    help="do not give the layer the tile-blocked copies of the bf16 experts")
    ap.add_argument("--event-every", type=int, default=8,
                    help="time the dominant launch with events on every N-th timed step")
    ap.add_argument("--no-probe-peaks", action="store_true",
                    help="skip measuring this GPU's MFMA and HBM peaks")
    ap.add_argument("--router-backward", action="store_true",
                    help="time moe_router_backward (training path) instead of the forward")
    ap.add_argument("--finish", action="store_true",
                    help="add the residual after the layer output (moe_forward_finish, "
                         "coefficients 1: the residual/bias-dropout-add), fused into the combine")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a 1 GiB streaming copy (counter calibration)")
    ap.add_argument("--write-traffic", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="summarise rocprofv3 counter runs into profiles/ (no GPU work)")
    ap.add_argument("--traffic-command", default="",
                    help="the command lines that produced the counter runs (recorded)")
    ap.add_argument("--write-mfma", metavar="COUNTER_CSV",
                    help="summarise a rocprofv3 --pmc run of MfmaUtil, MfmaFlopsBF16 and "
                         "GRBM_GUI_ACTIVE into profiles/ (no GPU work)")
    args = ap.parse_args()

    if args.write_traffic:
        write_traffic(args.workload, *args.write_traffic, args.traffic_command)
        return 0
    if args.write_mfma:
        write_mfma(args.workload, args.write_mfma, args.traffic_command)
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this layer is built and measured at EP=TP=1 on a single MI355X)", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy(1 << 30, 5)
        return 0
    if args.router_backward:
        return router_backward_bench(args)

    import numpy as np
    import torch
    import moe_inputs
    import mixture_experts_layer_steered_amd as moe

    wl = moe_inputs.WORKLOADS[args.workload]
    steps = args.steps if args.steps is not None else (300 if wl.T <= 64 else 20)
    warmup = args.warmup if args.warmup is not None else (30 if wl.T <= 64 else 3)
    # the oracle widens every touched expert's weights once per forward, so it
    # runs on whole batches (up to 8192 tokens), not on small chunks
    sample = args.cpu_sample if args.cpu_sample is not None else min(wl.T, 8192)

    print(f"[bench] generating {wl.label()}", file=sys.stderr, flush=True)
    inp = moe_inputs.generate(wl, seed=0)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")

    def dev_f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")

    T, H, E, k, I, Is = wl.T, wl.H, wl.E, wl.k, wl.I, wl.I_s
    params = moe.make_params(T, H, E, k, I, Is, wl.rsf, wl.limit, wl.scmoe, wl.eps, w4=wl.w4)
    x = dev_bf16(inp["x"])
    x_cur = dev_bf16(inp["x_cur"]) if wl.scmoe else None
    w4 = {}
    if wl.w4:  # W4A16 routed experts: packed codes, E4M3 scales, fp32 tensor scales
        w4 = dict(w_gate_up_q=torch.from_numpy(inp["w_gate_up_q"]).to("cuda"),
                  w_gate_up_scale=torch.from_numpy(inp["w_gate_up_scale"]).to("cuda"),
                  w_down_q=torch.from_numpy(inp["w_down_q"]).to("cuda"),
                  w_down_scale=torch.from_numpy(inp["w_down_scale"]).to("cuda"),
                  w_gate_up_tscale=dev_f32(inp["w_gate_up_tscale"]),
                  w_down_tscale=dev_f32(inp["w_down_tscale"]))
    dev = dict(w_router=dev_f32(inp["w_router"]), corr_bias=dev_f32(inp["corr_bias"]),
               w_gate_up=None if wl.w4 else dev_bf16(inp["w_gate_up"]),
               w_down=None if wl.w4 else dev_bf16(inp["w_down"]),
               ws_gate_up=dev_bf16(inp["ws_gate_up"]) if Is else None,
               ws_down=dev_bf16(inp["ws_down"]) if Is else None,
               gamma_pre=dev_f32(inp["gamma_pre"]) if wl.scmoe else None,
               gamma_post=dev_f32(inp["gamma_post"]) if wl.scmoe else None)
    # bf16 experts: their tile-blocked copies are written once here, before
    # any timing, as a weight-loading step (moe_pack_experts); the 256-row
    # tiles read them, the other tiles the row-major weights
    layout = "row_major"
    if not args.row_major_experts and H % 32 == 0 and I % 32 == 0 and Is % 32 == 0 and (
            Is or not wl.w4):
        if not wl.w4:  # W4A16 routed experts: the shared expert's copies only
            gu_n, dn_n = moe.moe_packed_experts_size(params)
            dev["w_gate_up_packed"] = torch.empty(gu_n, dtype=torch.int16, device="cuda")
            dev["w_down_packed"] = torch.empty(dn_n, dtype=torch.int16, device="cuda")
            moe.moe_pack_experts(params, dev["w_gate_up"], dev["w_down"],
                                 dev["w_gate_up_packed"], dev["w_down_packed"])
        if Is:
            ps = moe.make_params(T, H, 1, 1, Is, 0, wl.rsf, wl.limit, False, wl.eps)
            sgu_n, sdn_n = moe.moe_packed_experts_size(ps)
            dev["ws_gate_up_packed"] = torch.empty(sgu_n, dtype=torch.int16, device="cuda")
            dev["ws_down_packed"] = torch.empty(sdn_n, dtype=torch.int16, device="cuda")
            moe.moe_pack_experts(ps, dev["ws_gate_up"], dev["ws_down"],
                                 dev["ws_gate_up_packed"], dev["ws_down_packed"])
        torch.cuda.synchronize()
        layout = "row_major+tile_blocked" if not wl.w4 else "w4a16_codes+shared_tile_blocked"
    weights = moe.make_weights(**dev, **w4)
    ws = torch.empty(moe.moe_workspace_size(params), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")

    residual_bits = None
    fin = None
    if args.finish:
        residual_bits = moe_inputs.f32_to_bf16_bits(
            np.random.default_rng(1).standard_normal((T, H)).astype(np.float32))
        residual = dev_bf16(residual_bits)
        fin = moe.make_finish(residual, 1.0, 1.0)

    def forward(probes):
        if fin is not None:
            moe.moe_forward_finish(params, x, x_cur, weights, fin, out, probes, ws)
        else:
            moe.moe_forward(params, x, x_cur, weights, out, probes, ws)

    # one probed call to learn the routing (touched experts) for the byte count
    forward(moe.make_probes(expert_offsets=offsets))
    torch.cuda.synchronize()
    counts = np.diff(offsets.cpu().numpy())
    touched = int(np.sum(counts > 0))

    peaks = None
    if not args.no_probe_peaks:
        print("[bench] measuring this GPU's MFMA and HBM peaks", file=sys.stderr, flush=True)
        peaks = measure_peaks(moe, torch)

    # the dominant launch is timed by events that moe_forward records around
    # it on every `every`-th timed step (each event is a packet in the
    # stream, which costs the next launch a few microseconds: sampling keeps
    # them out of most steps); at least one step is timed
    every = max(1, args.event_every)
    timed = list(range(0, steps, every))
    hip = HipEvents()
    evs = {i: (hip.create(), hip.create()) for i in timed}
    probes = {i: moe.make_probes(events={moe.MOE_EV_PERMUTE: a, moe.MOE_EV_GATE_UP: b})
              for i, (a, b) in evs.items()}

    print(f"[bench] warmup {warmup}, steps {steps}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        forward(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        forward(probes.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    gate_up_ms = sum(hip.elapsed_ms(a, b) for a, b in evs.values()) / len(evs)
    for a, b in evs.values():
        hip.destroy(a)
        hip.destroy(b)

    # algorithmic work of the dominant launch and of the whole layer
    hbm_bound = wl.T * k <= 64 * E   # about a row tile per expert or less: weight streaming
    # bytes of one routed expert's weights of R rows x K: bf16, or W4A16
    # codes (half a byte each), one E4M3 scale byte per row and 128 columns
    # and the fp32 tensor scale
    def wbytes(R, K):
        return R * K // 2 + R * (K // 128) + 4 if wl.w4 else R * K * 2
    gu_bytes = touched * wbytes(2 * I, H) + T * H * 2 + T * k * I * 2
    gu_flops = 2 * T * k * H * 2 * I + 2 * T * H * 2 * Is
    layer_bytes = (touched * (wbytes(2 * I, H) + wbytes(H, I)) + 3 * Is * H * 2 + E * H * 4 + E * 4
                   + T * H * 2 * (2 if wl.scmoe else 1) + T * H * 2
                   + (T * H * 2 if args.finish else 0))
    layer_flops = 2 * T * k * H * 3 * I + 2 * T * H * 3 * Is
    router_flops = 2 * T * H * E
    traffic = committed_traffic(wl.label())
    if hbm_bound:
        achieved = gu_bytes / (gate_up_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": "grouped gate_up + SwiGLU (routed experts; the shared expert "
                              "runs beside the routing kernels on a second stream)",
                    "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_ms": round(gate_up_ms, 5),
                    "launches_timed": len(evs)}
    else:
        achieved = gu_flops / (gate_up_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                    "traffic": traffic,
                    "kernel": ("grouped gate_up + SwiGLU (routed W4A16 experts unpacked in "
                               "the tile, then the bf16 shared expert: two launches)"
                               if wl.w4 else
                               "grouped gate_up + SwiGLU (routed + shared, one launch)"),
                    "algorithmic_flops_per_launch": gu_flops, "avg_launch_ms": round(gate_up_ms, 5),
                    "launches_timed": len(evs)}
    if peaks is not None:
        mp = peaks["hbm_read_gbs"] if hbm_bound else peaks["mfma_bf16_tflops"]
        roofline["measured_peak"] = mp
        roofline["frac_measured"] = round(achieved / mp, 4)
    s_step = ms_per_step * 1e-3
    layer = {"tokens_per_s": round(T / s_step, 1),
             "GB_per_s": round(layer_bytes / s_step / 1e9, 1),
             "hbm_frac": round(layer_bytes / s_step / 1e9 / HBM_PEAK_GBS, 4),
             "TFLOP_per_s": round((layer_flops + router_flops) / s_step / 1e12, 1),
             "mfma_frac": round((layer_flops + router_flops) / s_step / 1e12 / BF16_PEAK_TFLOPS, 4),
             "experts_touched": touched, "max_over_mean_count": round(float(counts.max() / counts.mean()), 2)}
    if peaks is not None:
        layer["hbm_frac_measured"] = round(layer_bytes / s_step / 1e9 / peaks["hbm_read_gbs"], 4)
        layer["mfma_frac_measured"] = round((layer_flops + router_flops) / s_step / 1e12
                                            / peaks["mfma_bf16_tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] cpu oracle on {sample} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp, sample, args.cpu_seconds, residual_bits)

    line = {
        "metric": METRIC, "value": round(T / s_step, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.label(), "T": T, "H": H, "E": E, "k": k, "I": I, "I_shared": Is,
                   "routed_scaling_factor": wl.rsf, "swiglu_limit": wl.limit,
                   "scmoe": wl.scmoe, "seed": 0, "parallelism": "ep1_tp1",
                   "finish": "residual_add" if args.finish else None,
                   "expert_layout": layout},
        "roofline": roofline, "cpu_baseline": cpu, "layer": layer, "measured_peaks": peaks,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
