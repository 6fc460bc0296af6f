"""Routed mixture-of-experts MLP forward for MI355X (gfx950): Python binding.

A thin ctypes layer over libmoe.so (the C ABI in include/moe.h).  Every
function has the C name, takes torch tensors (device memory) or None for a
NULL pointer, marshals them to pointers, enqueues on the current (or given)
HIP stream and raises MoeError on a non-OK status.  All arithmetic happens
in the library's HIP kernels; there is no other implementation behind
these names.  The library is loaded on the first call (so that the build
module, python -m mixture_experts_layer_steered_amd.build, can run on a
fresh checkout); that call raises ImportError if it has not been built.

bf16 tensors may be torch.bfloat16 or torch.int16/uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, Structure, c_char_p, c_double, c_float, c_int, c_int32, c_int64,
                    c_size_t, c_void_p)

# torch first, at import: its bundled HIP runtime (soname libamdhip64.so.7)
# is then the one libmoe.so binds to whenever it is loaded in this process,
# so one runtime serves both (streams and device pointers are objects of
# that runtime).  A process that loads libmoe.so before importing torch
# binds the system runtime instead, and torch's tensors are not its own.
import torch  # noqa: F401,E402

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_DEVICE = 4
MOE_MAX_TOP_K = 16
MOE_MAX_EXPERTS = 1024
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_status_name(status)}: {detail}")


class moe_params(Structure):
    _fields_ = [
        ("T", c_int64), ("H", c_int32), ("E", c_int32), ("k", c_int32), ("I", c_int32),
        ("I_shared", c_int32), ("routed_scaling_factor", c_float), ("swiglu_limit", c_float),
        ("scmoe", c_int32), ("norm_eps", c_float), ("w4", c_int32),
    ]


class moe_weights(Structure):
    _fields_ = [(n, c_void_p) for n in (
        "w_router", "corr_bias", "w_gate_up", "w_down", "ws_gate_up", "ws_down",
        "gamma_pre", "gamma_post", "w_gate_up_q", "w_gate_up_scale", "w_down_q",
        "w_down_scale", "w_gate_up_tscale", "w_down_tscale", "w_gate_up_packed",
        "w_down_packed", "ws_gate_up_packed", "ws_down_packed")]


class moe_finish(Structure):
    _fields_ = [("residual", c_void_p), ("out_scale", c_float), ("residual_scale", c_float),
                ("post_norm", c_int32)]


MOE_EV_BEGIN, MOE_EV_PRENORM, MOE_EV_ROUTER, MOE_EV_PERMUTE = 0, 1, 2, 3
MOE_EV_GATE_UP, MOE_EV_DOWN, MOE_EV_COMBINE, MOE_EV_COUNT = 4, 5, 6, 7


class moe_probes(Structure):
    _fields_ = [(n, c_void_p) for n in (
        "topk_ids", "topk_w", "expert_offsets", "sorted_token", "inv_pos", "xr", "logits", "h",
        "y", "h_shared", "y_shared")] + [("events", c_void_p * MOE_EV_COUNT)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m mixture_experts_layer_steered_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    st = c_int
    P = POINTER(moe_params)
    sig = {
        "moe_workspace_size": (st, [P, POINTER(c_size_t)]),
        "moe_router_topk": (st, [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_size_t, c_void_p]),
        "moe_permute": (st, [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_size_t, c_void_p]),
        "moe_grouped_gemm_workspace_size": (st, [c_int32, c_int64, c_int32, c_int32,
                                                 POINTER(c_size_t)]),
        "moe_grouped_swiglu_gemm": (st, [c_int32, c_int64, c_int32, c_int32, c_float, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_size_t, c_void_p]),
        "moe_combine": (st, [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p]),
        "moe_forward": (st, [P, c_void_p, c_void_p, POINTER(moe_weights), c_void_p,
                             POINTER(moe_probes), c_void_p, c_size_t, c_void_p]),
        "moe_combine_finish": (st, [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    POINTER(moe_finish), c_void_p, c_void_p]),
        "moe_forward_finish": (st, [P, c_void_p, c_void_p, POINTER(moe_weights),
                                    POINTER(moe_finish), c_void_p, POINTER(moe_probes), c_void_p,
                                    c_size_t, c_void_p]),
        "moe_forward_noalloc": (st, [P, c_void_p, c_void_p, POINTER(moe_weights), c_void_p,
                                     POINTER(moe_probes), c_void_p]),
        "moe_router_backward_workspace_size": (st, [P, POINTER(c_size_t)]),
        "moe_router_backward": (st, [P, c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "moe_w4_dequantize": (st, [c_void_p, c_void_p, c_void_p, c_int32, c_int64, c_int32,
                                   c_void_p, c_void_p]),
        "moe_packed_experts_size": (st, [P, POINTER(c_int64), POINTER(c_int64)]),
        "moe_pack_experts": (st, [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
        "moe_probe_mfma_bf16": (st, [c_int32, c_int32, c_void_p, POINTER(c_double),
                                     c_void_p]),
        "moe_probe_hbm_read": (st, [c_void_p, c_int64, c_int32, c_void_p, c_void_p]),
        "moe_status_string": (c_char_p, [c_int]),
        "moe_last_error": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (loaded on first use; ImportError if missing)."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = _load()
    return _lib_handle


EXPORTED = ("moe_workspace_size", "moe_router_topk", "moe_permute",
            "moe_grouped_gemm_workspace_size", "moe_grouped_swiglu_gemm", "moe_combine",
            "moe_combine_finish", "moe_forward", "moe_forward_finish", "moe_forward_noalloc",
            "moe_router_backward_workspace_size", "moe_router_backward", "moe_w4_dequantize",
            "moe_packed_experts_size", "moe_pack_experts", "moe_probe_mfma_bf16", "moe_probe_hbm_read", "moe_status_string", "moe_last_error")


def _status_name(s: int) -> str:
    return lib().moe_status_string(s).decode()


def _check(s: int) -> None:
    if s != MOE_OK:
        raise MoeError(s, lib().moe_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    """Size of a workspace tensor; a raw integer pointer carries no size."""
    if t is None or isinstance(t, int):
        return 0
    return t.numel() * t.element_size()


def make_params(T, H, E, k, I, I_shared, routed_scaling_factor, swiglu_limit, scmoe=False,
                norm_eps=1e-6, w4=False) -> moe_params:
    return moe_params(int(T), int(H), int(E), int(k), int(I), int(I_shared),
                      float(routed_scaling_factor), float(swiglu_limit), int(bool(scmoe)),
                      float(norm_eps), int(bool(w4)))


def moe_workspace_size(params: moe_params) -> int:
    n = c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def moe_router_topk(params, x, w_router, corr_bias, topk_ids, topk_w, ws, stream=None):
    _check(lib().moe_router_topk(ctypes.byref(params), _ptr(x), _ptr(w_router), _ptr(corr_bias),
                                _ptr(topk_ids), _ptr(topk_w), _ptr(ws), _nbytes(ws),
                                _stream(stream)))


def moe_permute(params, topk_ids, expert_offsets, sorted_token, inv_pos, ws, stream=None,
                x=None, x_perm=None):
    _check(lib().moe_permute(ctypes.byref(params), _ptr(topk_ids), _ptr(x), _ptr(expert_offsets),
                            _ptr(sorted_token), _ptr(inv_pos), _ptr(x_perm), _ptr(ws),
                            _nbytes(ws), _stream(stream)))


def moe_grouped_gemm_workspace_size(n_groups, M_total, H, I) -> int:
    n = c_size_t(0)
    _check(lib().moe_grouped_gemm_workspace_size(int(n_groups), int(M_total), int(H), int(I),
                                                ctypes.byref(n)))
    return n.value


def moe_grouped_swiglu_gemm(n_groups, M_total, H, I, swiglu_limit, a, row_index, group_offsets,
                            w_gate_up, w_down, h, y, ws, stream=None):
    _check(lib().moe_grouped_swiglu_gemm(int(n_groups), int(M_total), int(H), int(I),
                                        float(swiglu_limit), _ptr(a), _ptr(row_index),
                                        _ptr(group_offsets), _ptr(w_gate_up), _ptr(w_down),
                                        _ptr(h), _ptr(y), _ptr(ws), _nbytes(ws),
                                        _stream(stream)))


def moe_combine(params, y_perm, topk_w, inv_pos, y_shared, gamma_post, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(params), _ptr(y_perm), _ptr(topk_w), _ptr(inv_pos),
                            _ptr(y_shared), _ptr(gamma_post), _ptr(out), _stream(stream)))


def make_finish(residual, out_scale=1.0, residual_scale=1.0, post_norm=False) -> moe_finish:
    """The residual add after the layer output (moe_finish in moe.h)."""
    return moe_finish(_ptr(residual), out_scale, residual_scale, int(bool(post_norm)))


def moe_combine_finish(params, y_perm, topk_w, inv_pos, y_shared, gamma_post, fin, out,
                       stream=None):
    f = ctypes.byref(fin) if fin is not None else None
    _check(lib().moe_combine_finish(ctypes.byref(params), _ptr(y_perm), _ptr(topk_w),
                                   _ptr(inv_pos), _ptr(y_shared), _ptr(gamma_post), f, _ptr(out),
                                   _stream(stream)))


def make_weights(w_router, corr_bias, w_gate_up, w_down, ws_gate_up=None, ws_down=None,
                 gamma_pre=None, gamma_post=None, w_gate_up_q=None, w_gate_up_scale=None,
                 w_down_q=None, w_down_scale=None, w_gate_up_tscale=None,
                 w_down_tscale=None, w_gate_up_packed=None, w_down_packed=None,
                 ws_gate_up_packed=None, ws_down_packed=None) -> moe_weights:
    """Weights of one layer; the W4A16 arrays (*_q codes, *_scale E4M3
    bytes, *_tscale fp32 tensor scales) replace w_gate_up / w_down when
    given; *_packed are the tile-blocked copies of moe_pack_experts."""
    return moe_weights(*[_ptr(t) for t in (w_router, corr_bias, w_gate_up, w_down, ws_gate_up,
                                           ws_down, gamma_pre, gamma_post, w_gate_up_q,
                                           w_gate_up_scale, w_down_q, w_down_scale,
                                           w_gate_up_tscale, w_down_tscale, w_gate_up_packed,
                                           w_down_packed, ws_gate_up_packed, ws_down_packed)])


def make_probes(topk_ids=None, topk_w=None, expert_offsets=None, sorted_token=None,
                inv_pos=None, xr=None, logits=None, events=None, h=None, y=None,
                h_shared=None, y_shared=None) -> moe_probes:
    """`events`: dict {MOE_EV_*: raw hipEvent_t handle (int)}."""
    pr = moe_probes(*[_ptr(t) for t in (topk_ids, topk_w, expert_offsets, sorted_token,
                                        inv_pos, xr, logits, h, y, h_shared, y_shared)])
    for i, ev in (events or {}).items():
        pr.events[i] = ev
    return pr


def moe_forward(params, x_routed, x_shared, weights: moe_weights, out, probes=None, ws=None,
                stream=None):
    pr = ctypes.byref(probes) if probes is not None else None
    _check(lib().moe_forward(ctypes.byref(params), _ptr(x_routed), _ptr(x_shared),
                            ctypes.byref(weights), _ptr(out), pr, _ptr(ws), _nbytes(ws),
                            _stream(stream)))


def moe_forward_finish(params, x_routed, x_shared, weights: moe_weights, fin, out, probes=None,
                       ws=None, stream=None):
    f = ctypes.byref(fin) if fin is not None else None
    pr = ctypes.byref(probes) if probes is not None else None
    _check(lib().moe_forward_finish(ctypes.byref(params), _ptr(x_routed), _ptr(x_shared),
                                   ctypes.byref(weights), f, _ptr(out), pr, _ptr(ws), _nbytes(ws),
                                   _stream(stream)))


def moe_forward_noalloc(params, x_routed, x_shared, weights: moe_weights, out, probes=None,
                        stream=None):
    """moe_forward on the library's fixed scratch (no workspace argument)."""
    pr = ctypes.byref(probes) if probes is not None else None
    _check(lib().moe_forward_noalloc(ctypes.byref(params), _ptr(x_routed), _ptr(x_shared),
                                     ctypes.byref(weights), _ptr(out), pr, _stream(stream)))


def moe_w4_dequantize(q, scale, out, n_groups, rows, K, stream=None, tscale=None):
    """W4A16 codes [n_groups, rows, K/2], E4M3 scales [n_groups, K/128, rows]
    and optional fp32 tensor scales [n_groups] -> bf16 bits [n_groups, rows,
    K] in `out`."""
    _check(lib().moe_w4_dequantize(_ptr(q), _ptr(scale), _ptr(tscale), int(n_groups), int(rows),
                                   int(K), _ptr(out), _stream(stream)))


def moe_packed_experts_size(params: moe_params):
    """(gate_up, down) element counts of the tile-blocked expert copies."""
    gu, dn = c_int64(0), c_int64(0)
    _check(lib().moe_packed_experts_size(ctypes.byref(params), ctypes.byref(gu),
                                         ctypes.byref(dn)))
    return gu.value, dn.value


def moe_pack_experts(params, w_gate_up, w_down, gate_up_packed, down_packed, stream=None):
    """Write the tile-blocked copies of the bf16 routed experts (sizes from
    moe_packed_experts_size) for moe_weights' *_packed fields."""
    _check(lib().moe_pack_experts(ctypes.byref(params), _ptr(w_gate_up), _ptr(w_down),
                                  _ptr(gate_up_packed), _ptr(down_packed), _stream(stream)))


def moe_router_backward_workspace_size(params: moe_params) -> int:
    n = c_size_t(0)
    _check(lib().moe_router_backward_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def moe_router_backward(params, grad_logits, x, w_router, grad_x=None, grad_w=None, grad_b=None,
                        ws=None, stream=None, strides=None):
    """Gradients of the router GEMM.  `grad_logits` is a float32 tensor
    [T, E] with any strides (an expanded one is read as it is), or a raw
    pointer with `strides` = (row, column) in elements."""
    if strides is None:
        strides = tuple(grad_logits.stride()) if grad_logits is not None else (0, 0)
    _check(lib().moe_router_backward(ctypes.byref(params), _ptr(grad_logits), int(strides[0]),
                                    int(strides[1]), _ptr(x), _ptr(w_router), _ptr(grad_x),
                                    _ptr(grad_w), _ptr(grad_b), _ptr(ws), _nbytes(ws),
                                    _stream(stream)))


def moe_probe_mfma_bf16(workgroups, iters, sink, stream=None) -> float:
    """Enqueue the bf16 MFMA throughput probe; returns the flops enqueued."""
    f = c_double(0.0)
    _check(lib().moe_probe_mfma_bf16(int(workgroups), int(iters), _ptr(sink), ctypes.byref(f),
                                     _stream(stream)))
    return f.value


def moe_probe_hbm_read(src, nbytes, workgroups, sink, stream=None) -> None:
    """Enqueue the HBM read-stream probe over nbytes of src."""
    _check(lib().moe_probe_hbm_read(_ptr(src), int(nbytes), int(workgroups), _ptr(sink),
                                    _stream(stream)))
